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
  float acc = 0.f;
  if (d.flags & kFlagVecFlat) {
    for (int64_t e = begin + threadIdx.x * 8; e < end; e += kEwThreads * 8) {
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

// ---------------------------------------------------------------------------
// K2: X0 = bf16(M / (||M|| + eps)) into the zero-padded rows_pad x cols_pad buffer
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
  const int64_t cp = d.cols_pad;
  const int64_t total = static_cast<int64_t>(d.rows_pad) * cp;
  const int64_t begin = (unit - prefix[i]) * kChunk;
  const int64_t end = begin + kChunk < total ? begin + kChunk : total;
  const bool vec = (d.flags & kFlagVecRows) != 0;
  uint16_t* x0 = d.x[0];
  for (int64_t e = begin + threadIdx.x * 8; e < end; e += kEwThreads * 8) {
    const int64_t r = e / cp, c0 = e - r * cp;
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
    gst<u32x4>(x0 + e, o);
  }
}

// ---------------------------------------------------------------------------
// K5: p <- p (1 - lr wd) - lr s O    (export_only: out <- O, unpadded)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kEwThreads) void k_apply(
    const MatDesc* __restrict__ descs, const int64_t* __restrict__ prefix, int n, int parity,
    float lr, float wd, int export_only) {
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  const int64_t total = d.rows * d.cols;
  const int64_t begin = (unit - prefix[i]) * kChunk;
  const int64_t end = begin + kChunk < total ? begin + kChunk : total;
  const uint16_t* o = d.x[parity];
  const int64_t cp = d.cols_pad, cols = d.cols;
  const float decay = 1.0f - lr * wd;
  const float step = lr * d.scale;
  if (d.flags & kFlagVecRows) {
    for (int64_t e = begin + threadIdx.x * 8; e < end; e += kEwThreads * 8) {
      const int64_t r = e / cols, c = e - r * cols;
      const u32x4 q = gld<u32x4>(o + r * cp + c);
      if (export_only) {
        gst<u32x4>(d.out + e, q);
      } else {
        f32x4 p0 = gld<f32x4>(d.param + e), p1 = gld<f32x4>(d.param + e + 4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          p0[2 * j] = fmaf(-step, __uint_as_float(q[j] << 16), p0[2 * j] * decay);
          p0[2 * j + 1] = fmaf(-step, __uint_as_float(q[j] & 0xffff0000u), p0[2 * j + 1] * decay);
          p1[2 * j] = fmaf(-step, __uint_as_float(q[2 + j] << 16), p1[2 * j] * decay);
          p1[2 * j + 1] = fmaf(-step, __uint_as_float(q[2 + j] & 0xffff0000u), p1[2 * j + 1] * decay);
        }
        gst<f32x4>(d.param + e, p0);
        gst<f32x4>(d.param + e + 4, p1);
      }
    }
  } else {
    for (int64_t e = begin + threadIdx.x; e < end; e += kEwThreads) {
      const int64_t r = e / cols, c = e - r * cols;
      const uint16_t q = gld<uint16_t>(o + r * cp + c);
      if (export_only) gst<uint16_t>(d.out + e, q);
      else gst<float>(d.param + e, fmaf(-step, bf2f(q), gld<float>(d.param + e) * decay));
    }
  }
}

// ---------------------------------------------------------------------------
// Newton-Schulz GEMMs on bf16 MFMA (v_mfma_f32_32x32x16_bf16)
//
// Workgroup tile 128 x 128, K step 64, 4 waves in a 2 x 2 grid, each wave
// 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.  Operands are staged in LDS as
// [row][k] with k contiguous; the 16-byte chunk c of row r is stored at
// chunk c ^ swz(r), so that the 32 rows an MFMA fragment read touches spread
// over all banks.  Two LDS buffers: the next K step's global loads are in
// flight while the current one is multiplied; one barrier per K step.
//
// An operand is "K-contiguous" (element (mn, k) at p[mn * ld + k]) or
// "MN-contiguous" (element (mn, k) at p[k * ld + mn]).  MN-contiguous tiles
// are transposed in registers (4 k x 8 mn blocks) on their way into LDS, so
// the inner loop is the same for every layout: the transpose of a tall
// matrix is never materialised.
// ---------------------------------------------------------------------------
constexpr int BM = kTile, BN = kTile, BK = kTileK;
constexpr int kLdsTile = BM * BK;  // bf16 elements per staged operand tile

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_idx(int row, int chunk) {
  return row * BK + ((chunk ^ swz(row)) << 3);
}

struct Opnd {
  const uint16_t* p;
  int64_t ld;
};

// global -> registers for one 128 x 64 operand tile
template <bool MN>
__device__ __forceinline__ void gload(const Opnd& op, int64_t mn0, int64_t k0, u32x4 (&r)[4]) {
  const int t = threadIdx.x;
  if constexpr (!MN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (t >> 3) + 32 * j, chunk = t & 7;
      r[j] = gld<u32x4>(op.p + (mn0 + row) * op.ld + k0 + chunk * 8);
    }
  } else {
    const int kq = t >> 4, mc = t & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = gld<u32x4>(op.p + (k0 + 4 * kq + j) * op.ld + mn0 + 8 * mc);
  }
}

// registers -> LDS (transposing MN-contiguous tiles)
template <bool MN>
__device__ __forceinline__ void lstore(uint16_t* s, const u32x4 (&r)[4]) {
  const int t = threadIdx.x;
  if constexpr (!MN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (t >> 3) + 32 * j, chunk = t & 7;
      *reinterpret_cast<u32x4*>(s + lds_idx(row, chunk)) = r[j];
    }
  } else {
    const int kq = t >> 4, mc = t & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // dword q of each k row holds mn = 2q (low half) and mn = 2q + 1 (high half)
      u32x2 lo, hi;
      lo.x = (r[0][q] & 0xffffu) | (r[1][q] << 16);
      lo.y = (r[2][q] & 0xffffu) | (r[3][q] << 16);
      hi.x = (r[0][q] >> 16) | (r[1][q] & 0xffff0000u);
      hi.y = (r[2][q] >> 16) | (r[3][q] & 0xffff0000u);
      const int row0 = 8 * mc + 2 * q;
      *reinterpret_cast<u32x2*>(s + lds_idx(row0, kq >> 1) + (kq & 1) * 4) = lo;
      *reinterpret_cast<u32x2*>(s + lds_idx(row0 + 1, kq >> 1) + (kq & 1) * 4) = hi;
    }
  }
}

// acc[bi][bj] += P(rows of this wave) * Q(cols of this wave)^T over one K step
__device__ __forceinline__ void mma_step(const uint16_t* sp, const uint16_t* sq,
                                         f32x16_t (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wr = w >> 1, wc = w & 1;
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int chunk = 2 * ks + (lane >> 5);
    bf16x8_t a[2], b[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const int row = 64 * wr + 32 * bi + (lane & 31);
      a[bi] = *reinterpret_cast<const bf16x8_t*>(sp + lds_idx(row, chunk));
    }
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int row = 64 * wc + 32 * bj + (lane & 31);
      b[bj] = *reinterpret_cast<const bf16x8_t*>(sq + lds_idx(row, chunk));
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
  }
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;
}

// acc += P[mp0 : mp0+128, :K] * Q[nq0 : nq0+128, :K]^T   (K a multiple of 64)
template <bool PMN, bool QMN>
__device__ __forceinline__ void gemm_tile(const Opnd& P, const Opnd& Q, int64_t mp0, int64_t nq0,
                                          int64_t K, uint16_t* smem, f32x16_t (&acc)[2][2]) {
  // buffer k holds P at smem + 2k * kLdsTile and Q right after it
  u32x4 rp[4], rq[4];
  gload<PMN>(P, mp0, 0, rp);
  gload<QMN>(Q, nq0, 0, rq);
  lstore<PMN>(smem, rp);
  lstore<QMN>(smem + kLdsTile, rq);
  __syncthreads();
  const int64_t kt_n = K / BK;
  for (int64_t kt = 0; kt < kt_n; ++kt) {
    uint16_t* cur = smem + static_cast<int>(kt & 1) * (2 * kLdsTile);
    uint16_t* nxt = smem + static_cast<int>((kt + 1) & 1) * (2 * kLdsTile);
    const bool more = kt + 1 < kt_n;
    if (more) {
      gload<PMN>(P, mp0, (kt + 1) * BK, rp);
      gload<QMN>(Q, nq0, (kt + 1) * BK, rq);
    }
    mma_step(cur, cur + kLdsTile, acc);
    if (more) {
      lstore<PMN>(nxt, rp);
      lstore<QMN>(nxt + kLdsTile, rq);
    }
    __syncthreads();
  }
}

// Position of accumulator element r of MFMA block (bi, bj) inside the 128 x 128 tile.
__device__ __forceinline__ void acc_pos(int bi, int bj, int r, int& row, int& col) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  row = 64 * (w >> 1) + 32 * bi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  col = 64 * (w & 1) + 32 * bj + (lane & 31);
}

// Symmetric store of a Gram-type tile (ti <= tj): the tile and its mirror.
// On a diagonal tile only the upper half (row <= col) is used for both
// positions, so the stored matrix is exactly symmetric.
//   GRAM2 == false:  out = bf16(acc)                          (A = X X^T)
//   GRAM2 == true:   C = a [row == col] + b A + c acc  (acc = A A), out = bf16(C),
//                    and out_lo = bf16(C - out) when out_lo is given.
template <bool GRAM2>
__device__ __forceinline__ void store_sym(const f32x16_t (&acc)[2][2], uint16_t* out,
                                          uint16_t* out_lo, const uint16_t* src, int64_t ld,
                                          int64_t ti, int64_t tj, float a, float b, float c) {
  const bool diag = ti == tj;
  const int64_t r0 = ti * BM, c0 = tj * BN;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint16_t h[4], l[4];
        int row = 0, col = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc_pos(bi, bj, 4 * g + q, row, col);
          float v = acc[bi][bj][4 * g + q];
          if constexpr (GRAM2) {
            const float diag_a = (diag && row == col) ? a : 0.f;
            v = fmaf(c, v, fmaf(b, bf2f(gld<uint16_t>(src + (r0 + row) * ld + c0 + col)), diag_a));
          }
          h[q] = f2bf(v);
          l[q] = f2bf(v - bf2f(h[q]));
        }
        acc_pos(bi, bj, 4 * g, row, col);  // rows row..row+3, one column
        if (!diag) {
#pragma unroll
          for (int q = 0; q < 4; ++q) gst<uint16_t>(out + (r0 + row + q) * ld + c0 + col, h[q]);
          u32x2 m;
          m.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
          m.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
          gst<u32x2>(out + (c0 + col) * ld + r0 + row, m);
          if (GRAM2 && out_lo) {
#pragma unroll
            for (int q = 0; q < 4; ++q) gst<uint16_t>(out_lo + (r0 + row + q) * ld + c0 + col, l[q]);
            m.x = l[0] | (static_cast<uint32_t>(l[1]) << 16);
            m.y = l[2] | (static_cast<uint32_t>(l[3]) << 16);
            gst<u32x2>(out_lo + (c0 + col) * ld + r0 + row, m);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (row + q <= col) {
              gst<uint16_t>(out + (r0 + row + q) * ld + c0 + col, h[q]);
              gst<uint16_t>(out + (c0 + col) * ld + r0 + row + q, h[q]);
              if (GRAM2 && out_lo) {
                gst<uint16_t>(out_lo + (r0 + row + q) * ld + c0 + col, l[q]);
                gst<uint16_t>(out_lo + (c0 + col) * ld + r0 + row + q, l[q]);
              }
            }
          }
        }
      }
}

__device__ __forceinline__ void decode_sym(int64_t u, int64_t t, int64_t& ti, int64_t& tj) {
  ti = 0;
  while (u >= t - ti) {
    u -= t - ti;
    ++ti;
  }
  tj = ti + u;
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

// K3a: A = X X^T for every matrix (upper tiles + mirror)
__global__ __launch_bounds__(kGemmThreads) void k_gram(const MatDesc* __restrict__ descs,
                                                       const int64_t* __restrict__ prefix, int n,
                                                       int64_t units, int parity) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kLdsTile];
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  int64_t ti, tj;
  decode_sym(unit - prefix[i], d.m_pad / BM, ti, tj);
  const Opnd X{d.x[parity], d.cols_pad};
  f32x16_t acc[2][2];
  zero_acc(acc);
  if (d.flags & kFlagTall)
    gemm_tile<true, true>(X, X, ti * BM, tj * BN, d.rows_pad, smem, acc);
  else
    gemm_tile<false, false>(X, X, ti * BM, tj * BN, d.cols_pad, smem, acc);
  store_sym<false>(acc, d.a, nullptr, nullptr, d.m_pad, ti, tj, 0.f, 0.f, 0.f);
}

// K3b: C = a I + b A + c A A  (A symmetric: A A = A A^T, a K-contiguous product).
// Folding a X into C (X' = C X) keeps the large cancelling terms of the
// polynomial inside one fp32 sum before the single bf16 rounding.
__global__ __launch_bounds__(kGemmThreads) void k_gram2(const MatDesc* __restrict__ descs,
                                                        const int64_t* __restrict__ prefix, int n,
                                                        int64_t units, float a, float b, float c) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kLdsTile];
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  int64_t ti, tj;
  decode_sym(unit - prefix[i], d.m_pad / BM, ti, tj);
  const Opnd A{d.a, d.m_pad};
  f32x16_t acc[2][2];
  zero_acc(acc);
  gemm_tile<false, false>(A, A, ti * BM, tj * BN, d.m_pad, smem, acc);
  store_sym<true>(acc, d.b, (d.flags & kFlagSplitC) ? d.blo : nullptr, d.a, d.m_pad, ti, tj, a, b, c);
}

// K4: X' = C X.  Wide (rows <= cols): X'[i][k] = sum_j C[i][j] X[j][k].
// Tall: the stored matrix is X^T, so X'^T = X^T C (C symmetric).
// Split matrices add the low part: X' = C_hi X + C_lo X.
__global__ __launch_bounds__(kGemmThreads) void k_xupdate(const MatDesc* __restrict__ descs,
                                                          const int64_t* __restrict__ prefix,
                                                          int n, int64_t units, int parity) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kLdsTile];
  const int64_t unit = xcd_remap(blockIdx.x, units);
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  int64_t ti, tj;
  decode_full(unit - prefix[i], d.rows_pad / BM, d.cols_pad / BN, ti, tj);
  const uint16_t* x = d.x[parity];
  uint16_t* xn = d.x[parity ^ 1];
  const int64_t ld = d.cols_pad;
  const bool split = (d.flags & kFlagSplitC) != 0;
  f32x16_t acc[2][2];
  zero_acc(acc);
  if (d.flags & kFlagTall) {
    gemm_tile<false, false>(Opnd{x, ld}, Opnd{d.b, d.m_pad}, ti * BM, tj * BN, d.m_pad, smem, acc);
    if (split)
      gemm_tile<false, false>(Opnd{x, ld}, Opnd{d.blo, d.m_pad}, ti * BM, tj * BN, d.m_pad, smem, acc);
  } else {
    gemm_tile<false, true>(Opnd{d.b, d.m_pad}, Opnd{x, ld}, ti * BM, tj * BN, d.m_pad, smem, acc);
    if (split)
      gemm_tile<false, true>(Opnd{d.blo, d.m_pad}, Opnd{x, ld}, ti * BM, tj * BN, d.m_pad, smem, acc);
  }
  const int64_t r0 = ti * BM, c0 = tj * BN;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int row, col;
        acc_pos(bi, bj, r, row, col);
        gst<uint16_t>(xn + (r0 + row) * ld + c0 + col, f2bf(acc[bi][bj][r]));
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

int launch_gram(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_gram, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, units, parity);
  return static_cast<int>(hipGetLastError());
}

int launch_gram2(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a, float b,
                 float c, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_gram2, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, units, a, b, c);
  return static_cast<int>(hipGetLastError());
}

int launch_xupdate(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                   void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_xupdate, dim3(static_cast<unsigned>(units)), dim3(kGemmThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, units, parity);
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
