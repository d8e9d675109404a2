// Fused Newton-Schulz iteration for small matrices (gfx950).
//
// One workgroup runs every iteration of one matrix with X, A and C resident
// in LDS: a step over many small matrices costs one launch for the whole
// iteration instead of three per iteration, and X does not travel to HBM
// between iterations.  The iteration is the newtonschulz5 routine of "Muon
// optimizer: matrix-aware LLM" (airosetta.com, implementation section) in
// the expanded form of "AdamW vs Muon" (adg.csdn.net, section "2. Newton-
// Schulz iteration"), with the rounding points of the tiled kernels
// (muon_gemm.h):
//   A  = bf16(X X^T)
//   C  = a I + b A + c A A,  C_hi = bf16(C),  C_lo = bf16(C - C_hi)
//   X' = bf16(C_hi X + C_lo X)
// each an fp32 MFMA accumulation rounded once to nearest-even.
//
// Eligible matrices (chosen on the host from the shape alone): short side
// m <= 128, both sides padded to 32, and X (m x n) plus two m x m buffers fit
// the 160 KB of LDS with every LDS row rounded up to 256 bytes.
//
// LDS layout: X as [m][ldx] (the logical m x n orientation: a tall matrix is
// transposed on the way in and out), P = A and later C_hi as [m][lda], Q =
// C_lo as [m][lda]; ldx, lda = the widths rounded up to 128 elements.  The
// 16-byte chunk c of row r sits at c ^ fsw(r), fsw(r) = 2 (r & 3) + 8 ((r >> 3)
// & 1), which makes both read forms conflict-free on the gfx950 LDS (64 banks
// of 4 bytes; a 16-byte read serves each half-wave in two cycles, lanes
// {0-3, 8-11, 20-23, 28-31} then the rest; a transposing 8-byte read serves
// 32 consecutive lanes per cycle; measured with the bank-conflict counter):
//   row fragments (lane l: row l & 15, chunk c + (l >> 4)): in each cycle the
//     even and the odd chunk of the pair land on all 16 bank groups;
//   column fragments (k rows 8 (l >> 4) + (l & 15) / 4, 32 bytes each): the 8
//     rows of one cycle have distinct fsw >> 1, i.e. distinct 32-byte spans.
#include <hip/hip_runtime.h>

#include <atomic>

#include "muon_device.h"

namespace muon {
namespace {

typedef short v4i16f __attribute__((ext_vector_type(4)));

constexpr int kFThreads = 512;  // 8 waves
constexpr int kFWaves = kFThreads / 64;

__device__ __forceinline__ int fsw(int r) { return ((r & 3) << 1) | (r & 8); }

// element offset of logical (r, c) in a swizzled LDS buffer with row length ld
__device__ __forceinline__ int spos(int r, int c, int ld) {
  return r * ld + (((c >> 3) ^ fsw(r)) << 3) + (c & 7);
}

// Row fragment: lane l holds row row0 + (l & 15), k = k0 + 8 (l >> 4) .. +7.
__device__ __forceinline__ bf16x8_t kfrag(const uint16_t* buf, int ld, int row0, int k0) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const bf16x8_t*>(buf + spos(row0 + (lane & 15), k0 + 8 * (lane >> 4), ld));
}

// Column fragment of a [k][mn] buffer: lane l holds column col0 + (l & 15),
// k = k0 + 8 (l >> 4) .. +7, assembled by two transposing reads (in each
// 16-lane group, lane 4a + b receives element b of the 8-byte pieces
// addressed by lanes a, a + 4, a + 8, a + 12).
__device__ __forceinline__ bf16x8_t cfrag(const uint16_t* buf, int ld, int col0, int k0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, i = lane & 15;
  const int k = k0 + 8 * g + (i >> 2), c = col0 + 4 * (i & 3);
  const v4i16f r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16f*)(buf + spos(k, c, ld)));
  const v4i16f r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16f*)(buf + spos(k + 4, c, ld)));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 x 8 transpose of 16-bit elements: out[s] element t = in[t] element s.
__device__ __forceinline__ void tr8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sh = 16 * (s & 1);
      const uint32_t lo = (in[2 * q][s >> 1] >> sh) & 0xffffu;
      const uint32_t hi = (in[2 * q + 1][s >> 1] >> sh) & 0xffffu;
      out[s][q] = lo | (hi << 16);
    }
}

// Global X buffer (stored orientation, rows_pad x cols_pad) <-> LDS X (m x n).
template <bool TO_LDS>
__device__ __forceinline__ void move_x(const MatDesc& d, uint16_t* g, uint16_t* X, int ldx, int M,
                                       int n) {
  if (!(d.flags & kFlagTall)) {  // stored = logical, [M][n]
    const int cpr = n >> 3, total = M * cpr;
    // 8 chunks per thread in flight: the loads' latency is paid once per batch
    constexpr int B = 8;
    for (int base = threadIdx.x; base < total; base += B * kFThreads) {
      u32x4 v[B];
      if constexpr (TO_LDS) {
#pragma unroll
        for (int j = 0; j < B; ++j) {
          const int idx = base + j * kFThreads;
          if (idx < total) {
            const int r = idx / cpr, c8 = idx - r * cpr;
            v[j] = gld<u32x4>(g + r * n + 8 * c8);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        const int idx = base + j * kFThreads;
        if (idx < total) {
          const int r = idx / cpr, c8 = idx - r * cpr;
          uint16_t* l = X + r * ldx + ((c8 ^ fsw(r)) << 3);
          if constexpr (TO_LDS) *reinterpret_cast<u32x4*>(l) = v[j];
          else gst<u32x4>(g + r * n + 8 * c8, *reinterpret_cast<const u32x4*>(l));
        }
      }
    }
  } else {  // stored [n][M] = X^T: 8 x 8 blocks transposed in registers
    const int bi = M >> 3;
    for (int idx = threadIdx.x; idx < bi * (n >> 3); idx += kFThreads) {
      const int ib = idx % bi, jb = idx / bi;
      u32x4 a[8], b[8];
      if constexpr (TO_LDS) {
#pragma unroll
        for (int t = 0; t < 8; ++t) a[t] = gld<u32x4>(g + (8 * jb + t) * M + 8 * ib);
        tr8(a, b);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 8 * ib + s;
          *reinterpret_cast<u32x4*>(X + r * ldx + ((jb ^ fsw(r)) << 3)) = b[s];
        }
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = 8 * ib + s;
          a[s] = *reinterpret_cast<const u32x4*>(X + r * ldx + ((jb ^ fsw(r)) << 3));
        }
        tr8(a, b);
#pragma unroll
        for (int t = 0; t < 8; ++t) gst<u32x4>(g + (8 * jb + t) * M + 8 * ib, b[t]);
      }
    }
  }
}

// LDS [M][lda] (swizzled) -> global M x M, row-major.
__device__ __forceinline__ void copy_sq(const uint16_t* P, int lda, uint16_t* g, int M) {
  const int cpr = M >> 3;
  for (int idx = threadIdx.x; idx < M * cpr; idx += kFThreads) {
    const int r = idx / cpr, c8 = idx - r * cpr;
    gst<u32x4>(g + r * M + 8 * c8,
               *reinterpret_cast<const u32x4*>(P + r * lda + ((c8 ^ fsw(r)) << 3)));
  }
}

// Upper-triangle 32 x 32 block t of an MB x MB grid -> (I <= J), row by row.
__device__ __forceinline__ void ublock(int t, int MB, int& I, int& J) {
  I = 0;
  while (t >= MB - I) {
    t -= MB - I;
    ++I;
  }
  J = I + t;
}

// Symmetric store of one 32 x 32 block's 16 values per lane (MFMA D layout:
// acc[p][q] holds column 32 J + 16 q + (lane & 15), rows 32 I + 16 p +
// 4 (lane >> 4) + e).  Only r <= c is written, at (r, c) and (c, r), so the
// stored matrix is exactly symmetric.
__device__ __forceinline__ void sym_store(uint16_t* P, int lda, int I, int J, const uint16_t (&h)[16]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 32 * I + 16 * p + 4 * (lane >> 4) + e, c = 32 * J + 16 * q + (lane & 15);
        if (r <= c) {
          const uint16_t v = h[(p * 2 + q) * 4 + e];
          P[spos(r, c, lda)] = v;
          P[spos(c, r, lda)] = v;
        }
      }
}

// acc = S[32 I ..][kb:ke] S[32 J ..][kb:ke]^T over row fragments of S (kb,
// ke multiples of 32, kb < ld).  The fragments of step k + 32 are read while
// the MFMAs of step k run.
__device__ __forceinline__ void gram_block(const uint16_t* S, int ld, int kb, int ke, int I, int J,
                                           f32x4_t (&acc)[2][2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[p][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16x8_t a0 = kfrag(S, ld, 32 * I, kb), a1 = kfrag(S, ld, 32 * I + 16, kb);
  bf16x8_t b0 = kfrag(S, ld, 32 * J, kb), b1 = kfrag(S, ld, 32 * J + 16, kb);
  for (int k0 = kb; k0 < ke; k0 += 32) {
    const int kn = k0 + 32 < ke ? k0 + 32 : k0;  // the last step re-reads itself
    const bf16x8_t na0 = kfrag(S, ld, 32 * I, kn), na1 = kfrag(S, ld, 32 * I + 16, kn);
    const bf16x8_t nb0 = kfrag(S, ld, 32 * J, kn), nb1 = kfrag(S, ld, 32 * J + 16, kn);
    acc[0][0] = mfma(a0, b0, acc[0][0]);
    acc[0][1] = mfma(a0, b1, acc[0][1]);
    acc[1][0] = mfma(a1, b0, acc[1][0]);
    acc[1][1] = mfma(a1, b1, acc[1][1]);
    a0 = na0, a1 = na1, b0 = nb0, b1 = nb1;
  }
}

// All ns_steps iterations of one matrix whose padded short side is M.
//
// Work split over the 8 waves: the Gram's upper-triangle 32 x 32 blocks,
// each over K / KS of the columns when there are few blocks (partial sums of
// the second half meet the first through the idle C_lo buffer); C's blocks;
// the X update by 32-column blocks.
template <int M>
__device__ void ns_matrix(const MatDesc& d, uint16_t* lds, const float* __restrict__ coeffs,
                          int n_coeffs, int ns_steps) {
  constexpr int MB = M / 32;                 // 32-row blocks per side
  constexpr int NBLK = MB * (MB + 1) / 2;    // upper-triangle blocks
  constexpr int KS = NBLK * 2 <= kFWaves ? 2 : 1;   // K split of the Gram
  constexpr int PER = (NBLK + kFWaves - 1) / kFWaves;
  constexpr int lda = (M + 127) & ~127;
  constexpr int RB = M / 16;                 // 16-row blocks of the X update
  static_assert(KS == 1 || NBLK * 1024 * 4 <= M * lda * 2, "Gram partials exceed C_lo");
  const int n = d.n_pad;
  const int ldx = (n + 127) & ~127;
  uint16_t* X = lds;
  uint16_t* P = X + M * ldx;
  uint16_t* Q = P + M * lda;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;

  move_x<true>(d, d.x[0], X, ldx, M, n);
  __syncthreads();
  for (int k = 0; k < ns_steps; ++k) {
    const int ci = n_coeffs == 1 ? 0 : k;
    const float ca = coeffs[3 * ci], cb = coeffs[3 * ci + 1], cc = coeffs[3 * ci + 2];
    const bool last = k == ns_steps - 1;
    // the iterate before the last goes to its ping-pong buffer (X0 is there already)
    if (last && k >= 1) move_x<false>(d, d.x[k & 1], X, ldx, M, n);

    // A = X X^T.  Work item u = w, w + 8, ...: block u % NBLK over K part
    // u / NBLK (with the K split there is a single round).
    static_assert(KS == 1 || NBLK * KS <= kFWaves, "one round when the K is split");
    for (int u0 = 0; u0 < NBLK * KS; u0 += kFWaves) {
      const int u = u0 + w;
      const bool active = u < NBLK * KS;
      const int t = u % NBLK, part = u / NBLK;
      int I = 0, J = 0;
      f32x4_t acc[2][2];
      float* pbuf = reinterpret_cast<float*>(Q) + t * 1024 + lane * 16;
      if (active) {
        ublock(t, MB, I, J);
        const int half = KS == 2 ? (((n >> 5) + 1) >> 1) << 5 : n;
        gram_block(X, ldx, part == 0 ? 0 : half, part == 0 ? half : n, I, J, acc);
        if (KS == 2 && part == 1) {
#pragma unroll
          for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4_t*>(pbuf + 4 * j) = acc[j >> 1][j & 1];
        }
      }
      if constexpr (KS == 2) __syncthreads();
      if (active && part == 0) {
        if constexpr (KS == 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j >> 1][j & 1] += *reinterpret_cast<const f32x4_t*>(pbuf + 4 * j);
        }
        uint16_t h[16];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) h[(p * 2 + q) * 4 + e] = f2bf(acc[p][q][e]);
        sym_store(P, lda, I, J, h);
      }
    }
    __syncthreads();
    if (last) copy_sq(P, lda, d.a, M);

    // C = a I + b A + c A A, kept in registers until every wave is done with A
    uint32_t hold[PER][16];
#pragma unroll
    for (int s = 0; s < PER; ++s) {
      const int t = w + kFWaves * s;
      if (t < NBLK) {
        int I, J;
        ublock(t, MB, I, J);
        f32x4_t acc[2][2];
        gram_block(P, lda, 0, M, I, J, acc);  // A symmetric: A A = A A^T
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 32 * I + 16 * p + 4 * (lane >> 4) + e, c = 32 * J + 16 * q + (lane & 15);
              const float av = bf2f(P[spos(r, c, lda)]);
              const float v = fmaf(cc, acc[p][q][e], fmaf(cb, av, r == c ? ca : 0.f));
              const uint16_t hi = f2bf(v);
              const uint16_t lo = f2bf(v - bf2f(hi));
              hold[s][(p * 2 + q) * 4 + e] = hi | (static_cast<uint32_t>(lo) << 16);
            }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < PER; ++s) {
      const int t = w + kFWaves * s;
      if (t < NBLK) {
        int I, J;
        ublock(t, MB, I, J);
        uint16_t h[16], l[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          h[e] = static_cast<uint16_t>(hold[s][e] & 0xffffu);
          l[e] = static_cast<uint16_t>(hold[s][e] >> 16);
        }
        sym_store(P, lda, I, J, h);
        sym_store(Q, lda, I, J, l);
      }
    }
    __syncthreads();
    if (last) {
      copy_sq(P, lda, d.b, M);
      copy_sq(Q, lda, d.blo, M);
    }

    // X' = C_hi X + C_lo X, one 32-column block of X at a time, in place:
    // each block is read and rewritten by one wave only.  Operands exchanged
    // (X columns first), so a lane ends up with four consecutive columns of
    // one row of X'.
    for (int jb = w; jb < (n >> 5); jb += kFWaves) {
      f32x4_t acc[RB][2];
#pragma unroll
      for (int ri = 0; ri < RB; ++ri) acc[ri][0] = acc[ri][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const uint16_t* Cp = part == 0 ? P : Q;
#pragma unroll
        for (int k0 = 0; k0 < M; k0 += 32) {
          const bf16x8_t x0 = cfrag(X, ldx, 32 * jb, k0), x1 = cfrag(X, ldx, 32 * jb + 16, k0);
#pragma unroll
          for (int ri = 0; ri < RB; ++ri) {
            const bf16x8_t cf = kfrag(Cp, lda, 16 * ri, k0);
            acc[ri][0] = mfma(x0, cf, acc[ri][0]);
            acc[ri][1] = mfma(x1, cf, acc[ri][1]);
          }
        }
      }
#pragma unroll
      for (int ri = 0; ri < RB; ++ri)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int r = 16 * ri + (lane & 15), c = 32 * jb + 16 * q + 4 * (lane >> 4);
          u32x2 v;
          v.x = pack2(acc[ri][q][0], acc[ri][q][1]);
          v.y = pack2(acc[ri][q][2], acc[ri][q][3]);
          *reinterpret_cast<u32x2*>(X + spos(r, c, ldx)) = v;
        }
    }
    __syncthreads();
  }
  move_x<false>(d, d.x[ns_steps & 1], X, ldx, M, n);
}

// One workgroup per matrix; every matrix of the launch has padded short side M.
template <int M>
__global__ __launch_bounds__(kFThreads) void k_ns_fused(const MatDesc* __restrict__ descs,
                                                        const float* __restrict__ coeffs,
                                                        int n_coeffs, int ns_steps) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  ns_matrix<M>(descs[blockIdx.x], lds, coeffs, n_coeffs, ns_steps);
}

template <int M>
int launch_m(const MatDesc* d, int n, const float* coeffs, int n_coeffs, int ns_steps,
             int lds_bytes, hipStream_t stream) {
  // the dynamic-LDS limit is raised once per device (the kernel needs up to
  // 160 KB); later calls on that device skip it
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  if (!done[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ns_fused<M>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLdsMax);
    if (e != hipSuccess) return static_cast<int>(e);
    done[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(k_ns_fused<M>, dim3(static_cast<unsigned>(n)), dim3(kFThreads),
                     static_cast<unsigned>(lds_bytes), stream, d, coeffs, n_coeffs, ns_steps);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_ns_fused(int m_pad, const MatDesc* d, int n, const float* coeffs, int n_coeffs,
                    int ns_steps, int lds_bytes, void* stream) {
  if (n <= 0) return 0;
  if (lds_bytes <= 0 || lds_bytes > kFusedLdsMax) return static_cast<int>(hipErrorInvalidValue);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (m_pad) {
    case 32: return launch_m<32>(d, n, coeffs, n_coeffs, ns_steps, lds_bytes, st);
    case 64: return launch_m<64>(d, n, coeffs, n_coeffs, ns_steps, lds_bytes, st);
    case 96: return launch_m<96>(d, n, coeffs, n_coeffs, ns_steps, lds_bytes, st);
    case 128: return launch_m<128>(d, n, coeffs, n_coeffs, ns_steps, lds_bytes, st);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace muon
