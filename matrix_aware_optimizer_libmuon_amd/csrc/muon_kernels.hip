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
// Output tile TILE x TILE (128 or 256), K step 64, 4 waves in a 2 x 2 grid,
// each wave (TILE/2) x (TILE/2) = NB x NB MFMA blocks of 32 x 32 with fp32
// accumulators (256 of them per lane at TILE = 256, held in AGPRs).
//
// Operand tiles are loaded 16 bytes per lane into registers one K step
// ahead and stored into a double-buffered LDS; with K step 64 every global
// load covers whole 128-byte lines (K-contiguous rows are 128 bytes).  Each
// K step is four 16-deep MFMA substeps; the fragments of the next substep
// are read while the current one's MFMAs run.  Substep 0 stores the P part
// of the next step and loads the P part of the step after; substep 1 does
// the same for Q; one LDS barrier, before substep 3, publishes the next
// step (substep 3 reads its first fragments).
//
// An operand is "K-contiguous" (element (mn, k) at p[mn * ld + k]) or
// "MN-contiguous" (element (mn, k) at p[k * ld + mn]).
//   K-contiguous tiles sit in LDS as [mn][64 k] (128-byte rows); fragments
//     are 16-byte reads; the 16-byte chunk c of row r is stored at
//     c ^ ((r >> 1) & 7).  The LDS has 64 banks of 4 bytes and serves 16
//     lanes of a 16-byte access per cycle: the 16 rows one fragment read
//     touches per cycle then cover all banks once (rows of equal parity
//     share bank offsets and differ in the XOR term).
//   MN-contiguous tiles keep their memory layout, [k][TILE mn]; fragments
//     are assembled by the LDS transpose read (ds_read_b64_tr_b16: in each
//     16-lane group, lane 4a + b receives element b of the 8-byte blocks
//     addressed by lanes a, a + 4, a + 8, a + 12), so the transpose of a tall
//     matrix is never materialised.  The 16-byte chunk c of k row r is
//     stored at c ^ (2 (r & 3)).
// ---------------------------------------------------------------------------
constexpr int BK = 64;
constexpr int kStages = 2;

template <int TILE>
struct Geo {
  static constexpr int T = TILE;
  static constexpr int WT = TILE / 2;      // wave tile
  static constexpr int NB = WT / 32;       // 32x32 MFMA blocks per wave side
  static constexpr int TE = TILE * BK;     // bf16 elements of one staged operand tile
  static constexpr int LPT = TILE / 32;    // 16-byte loads per thread per operand tile
  static constexpr int LDS = kStages * 2 * TE * 2;  // bytes
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N global loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct Opnd {
  const uint16_t* p;
  int64_t ld;
};

// This thread's share of one operand's TILE x 64 tile: LPT pieces of 16
// bytes.  Piece q of K step kt is read at byte base + kt kstep + q qstride
// (uniform) + voff (this lane's offset, 32 bits) and stored at LDS element
// lds + q QL.  Keeping the per-lane part in one 32-bit register lets every
// load use a scalar base address.
template <bool MN, int TILE>
struct Feed {
  static constexpr int CPR = MN ? TILE / 8 : BK / 8;        // 16-byte chunks per LDS row
  static constexpr int RPQ = kGemmThreads / CPR;            // LDS rows per piece
  static constexpr int QL = RPQ * (MN ? TILE : BK);         // LDS elements per piece
  const char* base;
  int64_t qstride, kstep;
  uint32_t voff;
  int lds;
  __device__ __forceinline__ Feed(const Opnd& op, int64_t mn0) {
    const int t = threadIdx.x;
    const int row = t / CPR, c = t % CPR;
    const int64_t ldb = op.ld * 2;
    voff = static_cast<uint32_t>(row * ldb + 16 * c);
    qstride = RPQ * ldb;
    if constexpr (!MN) {
      base = reinterpret_cast<const char*>(op.p) + mn0 * ldb;
      kstep = BK * 2;
      lds = row * BK + ((c ^ ((row >> 1) & 7)) << 3);
    } else {
      base = reinterpret_cast<const char*>(op.p) + mn0 * 2;
      kstep = BK * ldb;
      lds = row * TILE + ((c ^ (2 * (row & 3))) << 3);
    }
  }
  __device__ __forceinline__ u32x4 load(int64_t kt, int q) const {
    const char* b = base + kt * kstep + q * qstride;
    return gld<u32x4>(reinterpret_cast<const uint16_t*>(b + voff));
  }
  __device__ __forceinline__ void store(uint16_t* tile, int q, const u32x4& v) const {
    *reinterpret_cast<u32x4*>(tile + lds + q * QL) = v;
  }
};

// MFMA fragment (32 rows from rowbase, k = 16 sub .. 16 sub + 15) of one operand tile.
template <bool MN, int TILE>
__device__ __forceinline__ bf16x8_t frag(const uint16_t* tile, int rowbase, int sub) {
  const int lane = threadIdx.x & 63;
  if constexpr (!MN) {
    const int row = rowbase + (lane & 31);
    const int c = (2 * sub + (lane >> 5)) ^ ((row >> 1) & 7);
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
// K step kt lives in LDS buffer kt & 1.  Instruction order inside step kt,
// pinned with scheduling barriers (one MFMA per slot, NB*NB slots per substep):
//   substep 0: fragment reads of substep 1; wait for the P registers of
//              step kt+1, store them into the other buffer (its last reader
//              finished before the previous barrier), then load P of kt+2
//   substep 1: fragment reads of substep 2; the same for Q
//   substep 2: fragment reads of substep 3
//   LDS barrier: step kt+1 is complete in LDS
//   substep 3: fragment reads of substep 0 of step kt+1
// MFMA blocks are walked column by column, so each B fragment is consumed
// at least 3 NB MFMAs after it was read.  Loads past the end re-read the
// last step (stored, never consumed): the body has no branches.
//
// SWAP = true accumulates the transposed blocks (MFMA operands exchanged), so
// each lane ends up holding four consecutive output columns of one row.
template <int TILE, bool PMN, bool QMN, bool SWAP = false>
__device__ __forceinline__ void gemm_tile(const Opnd& P, const Opnd& Q, int64_t mp0, int64_t nq0,
                                          int64_t K, uint16_t* smem,
                                          f32x16_t (&acc)[Geo<TILE>::NB][Geo<TILE>::NB]) {
  using G = Geo<TILE>;
  constexpr int NB = G::NB, LPT = G::LPT, SLOTS = NB * NB;
  // per-slot quotas: fragment reads first, then stores, then loads
  constexpr int RD = (2 * NB + SLOTS - 1) / SLOTS;
  const int w = threadIdx.x >> 6;
  const int rowA = G::WT * (w >> 1), rowB = G::WT * (w & 1);
  const Feed<PMN, TILE> fp(P, mp0);
  const Feed<QMN, TILE> fq(Q, nq0);
  u32x4 gp[LPT], gq[LPT];
  bf16x8_t fa0[NB], fb0[NB], fa1[NB], fb1[NB];
  const int64_t kt_n = K / BK;
  auto buf = [&](int64_t kt) { return smem + static_cast<int>(kt & 1) * (2 * G::TE); };
  auto mfma = [&](const bf16x8_t (&fa)[NB], const bf16x8_t (&fb)[NB], int bi, int bj) {
    acc[bi][bj] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[bj], fa[bi], acc[bi][bj], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bi], fb[bj], acc[bi][bj], 0, 0, 0);
  };
  // fragment read number r (0 .. 2 NB - 1) of substep `sub` from tile `t`
  auto rd = [&](bf16x8_t (&fa)[NB], bf16x8_t (&fb)[NB], const uint16_t* t, int sub, int r) {
    if (r < NB) fa[r] = frag<PMN, TILE>(t, rowA + 32 * r, sub);
    else fb[r - NB] = frag<QMN, TILE>(t + G::TE, rowB + 32 * (r - NB), sub);
  };

#pragma unroll
  for (int q = 0; q < LPT; ++q) gp[q] = fp.load(0, q);
#pragma unroll
  for (int q = 0; q < LPT; ++q) gq[q] = fq.load(0, q);
  vm_wait<0>();
#pragma unroll
  for (int q = 0; q < LPT; ++q) fp.store(smem, q, gp[q]);
#pragma unroll
  for (int q = 0; q < LPT; ++q) fq.store(smem + G::TE, q, gq[q]);
  {
    const int64_t k1 = kt_n > 1 ? 1 : 0;
#pragma unroll
    for (int q = 0; q < LPT; ++q) gp[q] = fp.load(k1, q);
#pragma unroll
    for (int q = 0; q < LPT; ++q) gq[q] = fq.load(k1, q);
  }
  lds_barrier();
#pragma unroll
  for (int r = 0; r < 2 * NB; ++r) rd(fa0, fb0, smem, 0, r);

  // store + reload of piece j (P pieces 0 .. LPT-1, then Q pieces) sits in
  // slot (3 SLOTS j) / (2 LPT) of substeps 0-2: one pair every 1.5 slots
  auto pair = [&](uint16_t* nxt, int64_t kn, int j) {
    if (j < LPT) {
      fp.store(nxt, j, gp[j]);
      gp[j] = fp.load(kn, j);
    } else {
      fq.store(nxt + G::TE, j - LPT, gq[j - LPT]);
      gq[j - LPT] = fq.load(kn, j - LPT);
    }
  };
  for (int64_t kt = 0; kt < kt_n; ++kt) {
    const uint16_t* cur = buf(kt);
    uint16_t* nxt = buf(kt + 1);
    const int64_t kn = kt + 2 < kt_n ? kt + 2 : kt_n - 1;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      if (sub == 3) lds_barrier();  // step kt+1 is complete in LDS
#pragma unroll
      for (int s = 0; s < SLOTS; ++s) {
        if (sub & 1) mfma(fa1, fb1, s % NB, s / NB);
        else mfma(fa0, fb0, s % NB, s / NB);
#pragma unroll
        for (int r = 0; r < RD; ++r) {
          const int rr = s * RD + r;
          if (rr < 2 * NB) {
            if (sub == 0) rd(fa1, fb1, cur, 1, rr);
            else if (sub == 1) rd(fa0, fb0, cur, 2, rr);
            else if (sub == 2) rd(fa1, fb1, cur, 3, rr);
            else rd(fa0, fb0, nxt, 0, rr);
          }
        }
        if (sub < 3) {
          const int g = sub * SLOTS + s;
#pragma unroll
          for (int jj = 0; jj < 2 * LPT; ++jj)
            if ((jj * 3 * SLOTS) / (2 * LPT) == g) pair(nxt, kn, jj);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  vm_wait<0>();
  lds_barrier();  // every wave is done with every buffer
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
// the value computed for (col, row).  Works on 4 x 4 blocks: the four 8-byte
// column pieces of the upper block (b, a) are read, transposed in registers
// and written as the columns of the lower block (a, b), a > b; a diagonal
// block keeps its upper half and mirrors it into its lower half.
template <int TILE>
__device__ __forceinline__ void symmetrize(uint16_t* T) {
  constexpr int U = TILE / 4;                 // 4 x 4 blocks per side
  constexpr int NBLK = U * (U + 1) / 2;       // blocks on or below the diagonal
  for (int idx = threadIdx.x; idx < NBLK; idx += kGemmThreads) {
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
__device__ __forceinline__ void store_sym(const f32x16_t (&acc)[Geo<TILE>::NB][Geo<TILE>::NB],
                                          uint16_t* smem, uint16_t* out, uint16_t* out_lo,
                                          const uint16_t* src, int64_t ld, int64_t ti, int64_t tj,
                                          float a, float b, float c) {
  constexpr int NB = Geo<TILE>::NB;
  const bool diag = ti == tj;
  const int64_t r0 = ti * TILE, c0 = tj * TILE;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rowA = Geo<TILE>::WT * (w >> 1), rowB = Geo<TILE>::WT * (w & 1);
  // GRAM2: every A value the tile needs, loaded up front (one memory round
  // trip instead of one per block).  A is symmetric, so A[r0+rr+e][c0+cc] =
  // A[c0+cc][r0+rr+e]: rows rr .. rr+3 of column cc are one 8-byte load.
  // (At TILE = 128 the loads stay next to their use: the extra registers
  // would cost the second resident block per CU.)
  constexpr bool kBatch = GRAM2 && TILE == kTileBig;
  u32x2 asrc[kBatch ? NB : 1][kBatch ? NB : 1][kBatch ? 4 : 1];
  if constexpr (kBatch) {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj < NB; ++bj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = rowA + 32 * bi + 8 * q + 4 * (lane >> 5), cc = rowB + 32 * bj + (lane & 31);
          asrc[bi][bj][q] = gld<u32x2>(src + (c0 + cc) * ld + r0 + rr);
        }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first use
  }
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
            u32x2 av;
            if constexpr (kBatch) av = asrc[bi][bj][q];
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
  // Stage the bf16 tile in LDS, row-major with 8-byte units XORed by the row
  // (unit u of row r at u ^ (r & 31): a staging write, 32 rows at one unit,
  // then covers all banks), and write it out as whole 16-byte row chunks.
  // Transposed blocks: lane holds row rowA + 32 bi + (lane & 31), columns
  // rowB + 32 bj + 8 q + 4 (lane >> 5) .. +3.
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rl = G::WT * (w >> 1) + (lane & 31);
  const int cl = G::WT * (w & 1) + 4 * (lane >> 5);
#pragma unroll
  for (int bi = 0; bi < G::NB; ++bi)
#pragma unroll
    for (int bj = 0; bj < G::NB; ++bj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 m;
        m.x = pack2(acc[bi][bj][4 * q], acc[bi][bj][4 * q + 1]);
        m.y = pack2(acc[bi][bj][4 * q + 2], acc[bi][bj][4 * q + 3]);
        const int r = rl + 32 * bi, u = (cl + 32 * bj + 8 * q) >> 2;
        *reinterpret_cast<u32x2*>(smem + r * TILE + ((u ^ (r & 31)) << 2)) = m;
      }
  lds_barrier();
  constexpr int CPR = TILE / 8;  // 16-byte chunks per row
#pragma unroll 4
  for (int idx = threadIdx.x; idx < TILE * CPR; idx += kGemmThreads) {
    const int r = idx / CPR, ch = idx % CPR;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(smem + r * TILE + (((2 * ch) ^ (r & 31)) << 2));
    const u32x2 hi = *reinterpret_cast<const u32x2*>(smem + r * TILE + (((2 * ch + 1) ^ (r & 31)) << 2));
    gst<u32x4>(xn + (ti * TILE + r) * ld + tj * TILE + 8 * ch, u32x4{lo.x, lo.y, hi.x, hi.y});
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
