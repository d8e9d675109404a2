// Internal structures shared by the host dispatcher and the gfx950 kernels.
//
// Every call builds one device descriptor table (one MatDesc per active
// matrix) plus, per phase, a prefix sum of that phase's work units (element
// chunks or output tiles) per matrix.  Each phase is then ONE launch over the
// sum of all matrices' units: a workgroup finds its matrix by binary search
// in the prefix array.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace muon {

// Output tile of the Newton-Schulz GEMMs and padding granule of a matrix's
// bf16 workspace buffers.  Each matrix belongs to one tile class: 256 x 256
// tiles when its short side is at least kBigMinM, else 128 x 128.  All X / A
// / C buffers are zero-padded to multiples of the class tile in both
// dimensions, so the GEMM kernels never need bounds checks: zero rows and
// columns of X keep producing exact zeros in A and X'.
constexpr int kTileSmall = 128;
constexpr int kTileBig = 256;
constexpr int kBigMinM = 1024;
// Small matrices whose whole iteration fits in LDS take the fused kernel
// (muon_fused.hip): both sides padded to kTileFused, short side at most
// kFusedMaxM, and X plus two m x m buffers (LDS rows rounded up to 128
// elements) within kFusedLdsMax bytes.
constexpr int kTileFused = 32;
constexpr int kFusedMaxM = 128;
constexpr int kFusedLdsMax = 160 * 1024;
// Elements handled by one workgroup of the elementwise phases.
constexpr int kChunk = 16384;
constexpr int kEwThreads = 256;
constexpr int kGemmThreads = 256;

enum Phase : int {
  kPhaseMomentumNorm = 0,
  kPhaseNormalize = 1,
  kPhaseGram = 2,
  kPhaseGram2 = 3,
  kPhaseXUpdate = 4,
  kPhaseApply = 5,
  kPhaseAdamW = 6,
  kPhaseFusedNS = 7,
  kNumPhases = 8
};

// flags of MatDesc
enum : uint32_t {
  kFlagTall = 1u,        // rows > cols: the iteration runs on the transpose
  kFlagGradBf16 = 2u,    // grad / input is bf16 (else fp32)
  kFlagVecFlat = 4u,     // param/grad/mom 16-byte aligned and rows*cols % 8 == 0
  kFlagVecRows = 8u,     // additionally cols % 8 == 0 (row-wise 8-vectors)
  kFlagSplitC = 16u,     // C kept as a bf16 hi + lo pair (short side <= kSplitMaxM)
  // step variants (muon_step_ex options)
  kFlagZeroCenter = 32u, // G <- G - column means (colsum / rows) before use
  kFlagNesterov = 64u,   // NS input mu M_new + (1 - mu) G
  kFlagNsFirst = 128u,   // NS on G, then M <- mu M + (1 - mu) O and the update uses M
};

// Matrices whose short side is at most this keep C = a I + b A + c A A as a
// pair of bf16 matrices (hi + lo) and run the X update as two MFMA passes.
// Their Frobenius error then stays well inside the bf16 budget; the extra
// pass is one 128-wide tile row, i.e. negligible work.
constexpr int kSplitMaxM = 128;

// One matrix, as the kernels see it.  144 bytes.
struct alignas(16) MatDesc {
  float* param;          // fp32 rows x cols (muon_step) / unused (orthogonalize)
  const void* grad;      // grad (muon_step) or input (orthogonalize)
  float* mom;            // fp32 momentum (muon_step) / unused
  uint16_t* out;         // orthogonalize: bf16 rows x cols output / unused
  uint16_t* x[2];        // ping-pong bf16 X buffers, rows_pad x cols_pad
  uint16_t* a;           // bf16 m_pad x m_pad Gram
  uint16_t* b;           // bf16 m_pad x m_pad C = a I + b A + c A A (high part)
  uint16_t* blo;         // bf16 low part C - bf16(C) when kFlagSplitC, else null
  double* nrm2;          // sum of squares of M
  int64_t rows, cols;
  int32_t rows_pad, cols_pad, m_pad, n_pad;
  uint32_t flags;
  float scale;           // update scale s
  int32_t rg_pad;        // rows per work unit of the normalise pass (over rows_pad)
  int32_t rg;            // rows per work unit of the apply pass (over rows)
  double* colsum;        // column sums of G (kFlagZeroCenter), cols doubles
  double inv_rows;       // 1 / rows
};
static_assert(sizeof(MatDesc) == 144, "descriptor size");

// Column-sum pass of zero-centering: one work unit = kColRows rows x
// kColCols columns of one matrix.
constexpr int kColRows = 256;
constexpr int kColCols = 2048;

// One AdamW tensor, as the kernel sees it.  64 bytes.  The per-tensor bias
// corrections are folded on the host: step_size = lr / (1 - beta1^t),
// inv_sqrt_c2 = 1 / sqrt(1 - beta2^t), decay = 1 - lr wd.
struct alignas(16) AdamDesc {
  float* param;
  const void* grad;
  float* m;
  float* v;
  int64_t numel;
  float step_size, inv_sqrt_c2, decay;
  uint32_t flags;        // kFlagGradBf16, kFlagVecFlat
  int64_t reserved;
};
static_assert(sizeof(AdamDesc) == 64, "AdamW descriptor size");

// kernel launchers (muon_kernels.hip); return hipError_t as int.  `hyper`,
// when not null, points to {lr, mu, wd} in device memory and replaces the
// scalar arguments (read by the kernels when they run).
int launch_momentum_norm(const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                         float mu, const float* hyper, int norm_only, void* stream);
int launch_normalize(const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                     float eps, float mu, const float* hyper, void* stream);
int launch_fill_zero(double* p, int64_t count, void* stream);
int launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, void* stream);
int launch_colsum(const MatDesc* d, const int64_t* prefix, int n, int64_t units, double* zero_from,
                  int64_t zero_count, void* stream);
// GEMM phases: `tile` is 128 or 256; every matrix of the launch is of that class
int launch_gram(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                int parity, void* stream);
int launch_gram2(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                 float a, float b, float c, void* stream);
int launch_xupdate(int tile, const MatDesc* d, const int64_t* prefix, int n, int64_t units,
                   int parity, void* stream);
int launch_apply(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                 float lr, float wd, float mu, const float* hyper, int export_only, void* stream);
int launch_adamw(const AdamDesc* d, const int64_t* prefix, int n, int64_t units, float beta1,
                 float beta2, float eps, void* stream);
// fused iteration (muon_fused.hip): one workgroup per descriptor d[0 .. n),
// all of padded short side m_pad (32, 64, 96 or 128); coeffs = 3 floats per
// step on the device; lds_bytes = the largest need among them
int launch_ns_fused(int m_pad, const MatDesc* d, int n, const float* coeffs, int n_coeffs,
                    int ns_steps, int lds_bytes, void* stream);

// fixed scratch of muon_step_noalloc (muon_noalloc.hip): the address of the
// current device's array (resolved once per device), and a copy of host bytes
// into device memory through kernel arguments (no staging buffer)
int noalloc_scratch(int dev, void** out);
int put_bytes(void* dst, const void* src, size_t bytes, void* stream);

// per-tile GEMM launchers (muon_gemm256.hip, muon_gemm128.hip)
int launch_gram_256(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                   void* stream);
int launch_gram2_256(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a,
                    float b, float c, void* stream);
int launch_xupdate_256(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                      void* stream);
int launch_gram_128(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                   void* stream);
int launch_gram2_128(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a,
                    float b, float c, void* stream);
int launch_xupdate_128(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                      void* stream);


}  // namespace muon
