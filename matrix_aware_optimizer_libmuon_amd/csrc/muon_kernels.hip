// gfx950 (CDNA4) kernels of the Muon step.
//
//   K1 momentum + Frobenius sum of squares   (HBM-bound, one fp64 atomic per workgroup)
//   K2 normalise + cast to bf16              (HBM-bound, writes the zero-padded X0)
//   K3a Gram      A = X X^T                  (muon_gemm.h)
//   K3b Gram^2    C = a I + b A + c A A      (muon_gemm.h)
//   K4  X update  X' = C X                   (muon_gemm.h)
//   K5 apply      p <- p (1 - lr wd) - lr s O (HBM-bound)
//   AdamW         the branch for the parameters Muon does not take (HBM-bound)
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

#include "muon_device.h"

namespace muon {

// ---------------------------------------------------------------------------
// K1: M <- mu M + (1 - mu) G, and the sum of squares of the NS input:
//   default          sum of M^2
//   kFlagNesterov    sum of (mu M + (1 - mu) G)^2
//   kFlagNsFirst /   sum of G^2, no momentum update (the momentum comes after
//   norm_only        the iteration, or there is none: orthogonalize)
// With kFlagZeroCenter, G is first replaced by G - colsum / rows.
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

// Column index of a flat element index, advanced by a fixed stride without
// a division per step.
struct ColWalk {
  int64_t c, sc, w;
  __device__ ColWalk(int64_t first, int64_t stride, int64_t width)
      : c(first % width), sc(stride % width), w(width) {}
  __device__ void next() {
    c += sc;
    if (c >= w) c -= w;
  }
};

// g[j] -= mean of column c + j, j < K.  The mean is formed in fp64 and
// rounded once, so a column of equal values centres to exact zeros.
template <int K>
__device__ __forceinline__ void center(float (&g)[K], const MatDesc& d, int64_t c) {
#pragma unroll
  for (int j = 0; j < K; ++j) g[j] -= static_cast<float>(gld<double>(d.colsum + c + j) * d.inv_rows);
}

// one element of K1; returns its contribution to the sum of squares
__device__ __forceinline__ float k1_elem(float& m, float g, float mu, float omu, bool update,
                                         bool nest) {
  if (!update) return g * g;
  m = fmaf(mu, m, omu * g);
  const float x = nest ? fmaf(mu, m, omu * g) : m;
  return x * x;
}

__global__ __launch_bounds__(kEwThreads) void k_momentum_norm(
    const MatDesc* __restrict__ descs, const int64_t* __restrict__ prefix, int n,
    float mu, float omu, const float* __restrict__ hyper, int norm_only) {
  __shared__ double red[4];
  if (hyper) {
    mu = gld<float>(hyper + 1);
    omu = 1.0f - mu;
  }
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  const int64_t total = d.rows * d.cols;
  const int64_t begin = (unit - prefix[i]) * kChunk;
  const int64_t end = begin + kChunk < total ? begin + kChunk : total;
  const bool gbf = (d.flags & kFlagGradBf16) != 0;
  const bool zc = (d.flags & kFlagZeroCenter) != 0;
  const bool nest = (d.flags & kFlagNesterov) != 0;
  const bool update = !norm_only && !(d.flags & kFlagNsFirst);
  constexpr int S = kEwThreads * 8;  // elements per block-wide vector step
  float acc = 0.f;
  // with zero-centering the 8-vector must stay in one row: cols % 8 == 0
  if ((d.flags & kFlagVecFlat) && (!zc || (d.flags & kFlagVecRows))) {
    int64_t e = begin + threadIdx.x * 8;
    ColWalk cw(zc ? e : 0, S, zc ? d.cols : 1);
    // two 8-element vectors in flight per thread
    for (; e + S < end; e += 2 * S) {
      float g0[8], g1[8];
      load8_src(d.grad, gbf, e, g0);
      load8_src(d.grad, gbf, e + S, g1);
      if (zc) {
        center<8>(g0, d, cw.c);
        cw.next();
        center<8>(g1, d, cw.c);
        cw.next();
      }
      if (!update) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(g0[j], g0[j], fmaf(g1[j], g1[j], acc));
      } else {
        f32x4 m0 = gld<f32x4>(d.mom + e), m1 = gld<f32x4>(d.mom + e + 4);
        f32x4 m2 = gld<f32x4>(d.mom + e + S), m3 = gld<f32x4>(d.mom + e + S + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a = m0[j], b = m1[j], c = m2[j], q = m3[j];
          acc += k1_elem(a, g0[j], mu, omu, true, nest);
          acc += k1_elem(b, g0[4 + j], mu, omu, true, nest);
          acc += k1_elem(c, g1[j], mu, omu, true, nest);
          acc += k1_elem(q, g1[4 + j], mu, omu, true, nest);
          m0[j] = a, m1[j] = b, m2[j] = c, m3[j] = q;
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
      if (zc) center<8>(g, d, cw.c);
      if (!update) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(g[j], g[j], acc);
      } else {
        f32x4 m0 = gld<f32x4>(d.mom + e), m1 = gld<f32x4>(d.mom + e + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a = m0[j], b = m1[j];
          acc += k1_elem(a, g[j], mu, omu, true, nest);
          acc += k1_elem(b, g[4 + j], mu, omu, true, nest);
          m0[j] = a, m1[j] = b;
        }
        gst<f32x4>(d.mom + e, m0);
        gst<f32x4>(d.mom + e + 4, m1);
      }
    }
  } else {
    int64_t e = begin + threadIdx.x;
    ColWalk cw(zc ? e : 0, kEwThreads, zc ? d.cols : 1);
    for (; e < end; e += kEwThreads, cw.next()) {
      float g[1] = {load1_src(d.grad, gbf, e)};
      if (zc) center<1>(g, d, cw.c);
      if (!update) {
        acc = fmaf(g[0], g[0], acc);
      } else {
        float m = gld<float>(d.mom + e);
        acc += k1_elem(m, g[0], mu, omu, true, nest);
        gst<float>(d.mom + e, m);
      }
    }
  }
  const double s = block_sum_256(static_cast<double>(acc), red);
  if (threadIdx.x == 0) unsafeAtomicAdd(d.nrm2, s);
}

// ---------------------------------------------------------------------------
// Zero-centering, first pass: column sums of G into colsum (fp64 sums and
// atomics).
// Block 0 of the launch is preceded by a fill kernel zeroing every colsum.
// One work unit = kColRows rows x kColCols columns; a thread owns 8 columns.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kEwThreads) void k_fill_zero_f64(double* p, int64_t count) {
  for (int64_t k = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x; k < count;
       k += static_cast<int64_t>(gridDim.x) * kEwThreads)
    p[k] = 0.0;
}

// Fill count 32-bit words with a value (the debug mode's NaN poisoning of the
// iteration buffers; a kernel, not a memset node, so it is safe in any stream).
__global__ __launch_bounds__(kEwThreads) void k_fill_u32(uint32_t* p, int64_t count, uint32_t value) {
  for (int64_t k = blockIdx.x * static_cast<int64_t>(kEwThreads) + threadIdx.x; k < count;
       k += static_cast<int64_t>(gridDim.x) * kEwThreads)
    p[k] = value;
}

__global__ __launch_bounds__(kEwThreads) void k_colsum(const MatDesc* __restrict__ descs,
                                                       const int64_t* __restrict__ prefix, int n) {
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  const int64_t ncc = (d.cols + kColCols - 1) / kColCols;
  const int64_t u = unit - prefix[i];
  const int64_t r0 = (u / ncc) * kColRows, c0 = (u % ncc) * kColCols;
  const int64_t r1 = r0 + kColRows < d.rows ? r0 + kColRows : d.rows;
  const bool gbf = (d.flags & kFlagGradBf16) != 0;
  if (d.flags & kFlagVecRows) {  // cols % 8 == 0 and 16-byte aligned rows
    const int64_t c = c0 + threadIdx.x * 8;
    if (c >= d.cols) return;
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int64_t r = r0; r < r1; ++r) {
      float g[8];
      load8_src(d.grad, gbf, r * d.cols + c, g);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += static_cast<double>(g[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) unsafeAtomicAdd(d.colsum + c + j, acc[j]);
  } else {
    for (int64_t c = c0 + threadIdx.x; c < c0 + kColCols && c < d.cols; c += kEwThreads) {
      double acc = 0.0;
      for (int64_t r = r0; r < r1; ++r) acc += static_cast<double>(load1_src(d.grad, gbf, r * d.cols + c));
      unsafeAtomicAdd(d.colsum + c, acc);
    }
  }
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
// K2: X0 = bf16(N / (||N|| + eps)) into the zero-padded rows_pad x cols_pad
// buffer, N the NS input: M (default), the input (orthogonalize), G
// (kFlagNsFirst; centered with kFlagZeroCenter) or mu M + (1 - mu) G
// (kFlagNesterov).  One work unit = rg_pad padded rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kEwThreads) void k_normalize(
    const MatDesc* __restrict__ descs, const int64_t* __restrict__ prefix, int n, float eps,
    float mu, const float* __restrict__ hyper) {
  if (hyper) mu = gld<float>(hyper + 1);
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const MatDesc& d = descs[i];
  const bool from_grad = d.mom == nullptr || (d.flags & kFlagNsFirst);  // N = G
  const bool nest = (d.flags & kFlagNesterov) != 0;                    // N = mu M + (1-mu) G
  const bool zc = (d.flags & kFlagZeroCenter) != 0;
  const bool gbf = (d.flags & kFlagGradBf16) != 0;
  const float omu = 1.0f - mu;
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
      const int64_t g = r * d.cols + c0;
      if (from_grad || nest) {
        load8_src(d.grad, gbf, g, v);
        if (zc) center<8>(v, d, c0);
      }
      if (nest) {
        const f32x4 m0 = gld<f32x4>(d.mom + g), m1 = gld<f32x4>(d.mom + g + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = fmaf(mu, m0[j], omu * v[j]);
          v[4 + j] = fmaf(mu, m1[j], omu * v[4 + j]);
        }
      } else if (!from_grad) {
        load8_src(d.mom, false, g, v);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = 0.f;
        if (r < d.rows && c0 + j < d.cols) {
          const int64_t g = r * d.cols + c0 + j;
          float gv[1] = {0.f};
          if (from_grad || nest) {
            gv[0] = load1_src(d.grad, gbf, g);
            if (zc) center<1>(gv, d, c0 + j);
          }
          v[j] = nest ? fmaf(mu, gld<float>(d.mom + g), omu * gv[0])
                      : (from_grad ? gv[0] : gld<float>(d.mom + g));
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack2(v[2 * j] * inv, v[2 * j + 1] * inv);
    gst<u32x4>(x0 + r * cp + c0, o);
  }
}

// ---------------------------------------------------------------------------
// K5: p <- p (1 - lr wd) - lr s O    (export_only: out <- O, unpadded);
// with kFlagNsFirst: M <- mu M + (1 - mu) O, then p <- p (1 - lr wd) - lr s M.
// One work unit = rg rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kEwThreads) void k_apply(
    const MatDesc* __restrict__ descs, const int64_t* __restrict__ prefix, int n, int parity,
    float lr, float wd, float mu, const float* __restrict__ hyper, int export_only) {
  if (hyper) {
    lr = gld<float>(hyper);
    mu = gld<float>(hyper + 1);
    wd = gld<float>(hyper + 2);
  }
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
  const bool after = !export_only && (d.flags & kFlagNsFirst);
  const float omu = 1.0f - mu;
  if (d.flags & kFlagVecRows) {
    constexpr int S = kEwThreads * 8;
    RowWalk p(r0, threadIdx.x * 8, S, cols);
    for (int64_t e = threadIdx.x * 8; e < count; e += S, p.next()) {
      const int64_t r = p.r, c = p.c, g = r * cols + c;
      const u32x4 q = gld<u32x4>(o + r * cp + c);
      if (export_only) {
        gst<u32x4>(d.out + g, q);
      } else {
        float u[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u[2 * j] = __uint_as_float(q[j] << 16);
          u[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
        }
        if (after) {
          f32x4 m0 = gld<f32x4>(d.mom + g), m1 = gld<f32x4>(d.mom + g + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            m0[j] = fmaf(mu, m0[j], omu * u[j]);
            m1[j] = fmaf(mu, m1[j], omu * u[4 + j]);
            u[j] = m0[j];
            u[4 + j] = m1[j];
          }
          gst<f32x4>(d.mom + g, m0);
          gst<f32x4>(d.mom + g + 4, m1);
        }
        f32x4 p0 = gld<f32x4>(d.param + g), p1 = gld<f32x4>(d.param + g + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p0[j] = fmaf(-step, u[j], p0[j] * decay);
          p1[j] = fmaf(-step, u[4 + j], p1[j] * decay);
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
      if (export_only) {
        gst<uint16_t>(d.out + g, q);
      } else {
        float u = bf2f(q);
        if (after) {
          u = fmaf(mu, gld<float>(d.mom + g), omu * u);
          gst<float>(d.mom + g, u);
        }
        gst<float>(d.param + g, fmaf(-step, u, gld<float>(d.param + g) * decay));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// AdamW (the branch for parameters Muon does not take), one work unit =
// kChunk elements of one tensor, all fp32 math:
//   p <- p decay;  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
//   p <- p - step_size m / (sqrt(v) inv_sqrt_c2 + eps)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void adamw_elem(float& p, float& m, float& v, float g, float b1,
                                           float b2, float eps, float decay, float step_size,
                                           float inv_sqrt_c2) {
  p *= decay;
  m = fmaf(b1, m, (1.0f - b1) * g);
  v = fmaf(b2, v, (1.0f - b2) * (g * g));
  p = fmaf(-step_size, m / fmaf(sqrtf(v), inv_sqrt_c2, eps), p);
}

__global__ __launch_bounds__(kEwThreads) void k_adamw(const AdamDesc* __restrict__ descs,
                                                      const int64_t* __restrict__ prefix, int n,
                                                      float b1, float b2, float eps) {
  const int64_t unit = blockIdx.x;
  const int i = find_matrix(prefix, n, unit);
  const AdamDesc& d = descs[i];
  const int64_t begin = (unit - prefix[i]) * kChunk;
  const int64_t end = begin + kChunk < d.numel ? begin + kChunk : d.numel;
  const bool gbf = (d.flags & kFlagGradBf16) != 0;
  const float decay = d.decay, step = d.step_size, isc = d.inv_sqrt_c2;
  if (d.flags & kFlagVecFlat) {
    for (int64_t e = begin + threadIdx.x * 8; e < end; e += kEwThreads * 8) {
      float g[8];
      load8_src(d.grad, gbf, e, g);
      f32x4 p0 = gld<f32x4>(d.param + e), p1 = gld<f32x4>(d.param + e + 4);
      f32x4 m0 = gld<f32x4>(d.m + e), m1 = gld<f32x4>(d.m + e + 4);
      f32x4 v0 = gld<f32x4>(d.v + e), v1 = gld<f32x4>(d.v + e + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = p0[j], m = m0[j], v = v0[j];
        adamw_elem(p, m, v, g[j], b1, b2, eps, decay, step, isc);
        p0[j] = p, m0[j] = m, v0[j] = v;
        p = p1[j], m = m1[j], v = v1[j];
        adamw_elem(p, m, v, g[4 + j], b1, b2, eps, decay, step, isc);
        p1[j] = p, m1[j] = m, v1[j] = v;
      }
      gst<f32x4>(d.param + e, p0);
      gst<f32x4>(d.param + e + 4, p1);
      gst<f32x4>(d.m + e, m0);
      gst<f32x4>(d.m + e + 4, m1);
      gst<f32x4>(d.v + e, v0);
      gst<f32x4>(d.v + e + 4, v1);
    }
  } else {
    for (int64_t e = begin + threadIdx.x; e < end; e += kEwThreads) {
      float p = gld<float>(d.param + e), m = gld<float>(d.m + e), v = gld<float>(d.v + e);
      adamw_elem(p, m, v, load1_src(d.grad, gbf, e), b1, b2, eps, decay, step, isc);
      gst<float>(d.param + e, p);
      gst<float>(d.m + e, m);
      gst<float>(d.v + e, v);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline int grid_ok(int64_t units) { return units > 0 && units < (int64_t(1) << 31); }

int launch_momentum_norm(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float mu,
                         const float* hyper, int norm_only, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_momentum_norm, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, mu, 1.0f - mu, hyper, norm_only);
  return static_cast<int>(hipGetLastError());
}

int launch_normalize(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float eps,
                     float mu, const float* hyper, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_normalize, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, eps, mu, hyper);
  return static_cast<int>(hipGetLastError());
}

int launch_fill_zero(double* p, int64_t count, void* stream) {
  if (count <= 0) return 0;
  const int64_t blocks = (count + kEwThreads - 1) / kEwThreads;
  hipLaunchKernelGGL(k_fill_zero_f64, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)),
                     dim3(kEwThreads), 0, static_cast<hipStream_t>(stream), p, count);
  return static_cast<int>(hipGetLastError());
}

int launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, void* stream) {
  if (count <= 0) return 0;
  const int64_t blocks = (count + kEwThreads - 1) / kEwThreads;
  hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                     dim3(kEwThreads), 0, static_cast<hipStream_t>(stream), p, count, value);
  return static_cast<int>(hipGetLastError());
}

int launch_colsum(const MatDesc* d, const int64_t* prefix, int n, int64_t units, double* zero_from,
                  int64_t zero_count, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t fill_blocks = (zero_count + kEwThreads - 1) / kEwThreads;
  hipLaunchKernelGGL(k_fill_zero_f64, dim3(static_cast<unsigned>(fill_blocks < 1024 ? fill_blocks : 1024)),
                     dim3(kEwThreads), 0, st, zero_from, zero_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  hipLaunchKernelGGL(k_colsum, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0, st, d, prefix, n);
  return static_cast<int>(hipGetLastError());
}

int launch_gram(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                int parity, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  return tile == kTileBig ? launch_gram_256(d, prefix, n, units, parity, stream)
                          : launch_gram_128(d, prefix, n, units, parity, stream);
}

int launch_gram2(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a,
                 float b, float c, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  return tile == kTileBig ? launch_gram2_256(d, prefix, n, units, a, b, c, stream)
                          : launch_gram2_128(d, prefix, n, units, a, b, c, stream);
}

int launch_xupdate(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                   int parity, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  return tile == kTileBig ? launch_xupdate_256(d, prefix, n, units, parity, stream)
                          : launch_xupdate_128(d, prefix, n, units, parity, stream);
}

int launch_apply(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                 float lr, float wd, float mu, const float* hyper, int export_only, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_apply, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, parity, lr, wd, mu, hyper,
                     export_only);
  return static_cast<int>(hipGetLastError());
}

int launch_adamw(const AdamDesc* d, const int64_t* prefix, int n, int64_t units, float beta1,
                 float beta2, float eps, void* stream) {
  if (!grid_ok(units)) return static_cast<int>(hipErrorInvalidConfiguration);
  hipLaunchKernelGGL(k_adamw, dim3(static_cast<unsigned>(units)), dim3(kEwThreads), 0,
                     static_cast<hipStream_t>(stream), d, prefix, n, beta1, beta2, eps);
  return static_cast<int>(hipGetLastError());
}

}  // namespace muon
