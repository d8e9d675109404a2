// Host side of libmuon: argument checks, workspace planning, the device
// descriptor table and the grouped launch sequence.  The C ABI is declared
// in include/muon.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "muon.h"
#include "muon_internal.h"

using namespace muon;

namespace {

thread_local std::string g_hip_detail;

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// workspace plan (a pure function of the shapes)
//
//   [ table: MatDesc[n] | 8 prefix arrays int64[n+1] | nrm2 double[n] |
//     NS coefficients float[3 * MUON_MAX_NS_STEPS] ] (256-aligned)
//   [ column sums: double[cols] per matrix ] (256-aligned; zero-centering only)
//   then, per matrix (all n, skipped ones included):
//   [ X0 | X1 ] rows_pad x cols_pad bf16 each, [ A | C ] m_pad x m_pad bf16 each,
//   and [ C_lo ] m_pad x m_pad bf16 when the short side is <= kSplitMaxM
// ---------------------------------------------------------------------------
// prefix arrays of the table: element chunks (flat / padded) over all active
// matrices, symmetric and full tile counts per tile class, row groups of the
// apply pass, and column-sum blocks (zero-centering matrices only)
enum { kPreFlat = 0, kPrePad = 1, kPreSymBig = 2, kPreFullBig = 3, kPreSymSmall = 4,
       kPreFullSmall = 5, kPreRows = 6, kPreCol = 7, kNumPrefix = 8 };

int64_t ceil_to(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// LDS bytes the fused kernel needs for an r x c matrix (0: not eligible).
int64_t fused_lds(int64_t r, int64_t c) {
  const int64_t m = ceil_to(std::min(r, c), kTileFused), n = ceil_to(std::max(r, c), kTileFused);
  if (m > kFusedMaxM) return 0;
  const int64_t bytes = 2 * (m * ceil_to(n, 128) + 2 * m * ceil_to(m, 128));
  return bytes <= kFusedLdsMax ? bytes : 0;
}

// Padding granule / kernel class of a matrix: 256 or 128 (tiled GEMM
// launches) or kTileFused (the whole iteration in one workgroup).
int tile_class(int64_t r, int64_t c) {
  if (std::min(r, c) >= kBigMinM) return kTileBig;
  return fused_lds(r, c) ? kTileFused : kTileSmall;
}

struct MatPlan {
  int64_t rows, cols, rows_pad, cols_pad, m_pad, n_pad;
  int tile;
  bool tall, split;
  size_t x_off[2], a_off, b_off, blo_off, colsum_off;
};

struct Plan {
  int64_t n = 0;
  size_t desc_off = 0, prefix_off[kNumPrefix] = {}, nrm2_off = 0, coeff_off = 0, table_bytes = 0;
  size_t colsum_off = 0;
  int64_t colsum_count = 0;           // doubles in the column-sum region
  size_t buf_off = 0;                 // start of the per-matrix X / A / C buffers
  size_t total = 0;
  std::vector<MatPlan> mats;
};

bool shape_ok(int64_t r, int64_t c) { return r >= 1 && c >= 1 && r <= MUON_MAX_DIM && c <= MUON_MAX_DIM; }

template <class GetShape>
bool make_plan(int64_t n, GetShape shape, Plan& plan) {
  plan = Plan();
  plan.n = n;
  plan.desc_off = 0;
  size_t off = static_cast<size_t>(n) * sizeof(MatDesc);
  for (int k = 0; k < kNumPrefix; ++k) {
    plan.prefix_off[k] = off;
    off += static_cast<size_t>(n + 1) * sizeof(int64_t);
  }
  plan.nrm2_off = off;
  off += static_cast<size_t>(n) * sizeof(double);
  plan.coeff_off = off;
  off += 3 * MUON_MAX_NS_STEPS * sizeof(float);
  plan.table_bytes = align_up(off, kAlign);
  plan.mats.resize(static_cast<size_t>(n));
  plan.colsum_off = plan.table_bytes;
  for (int64_t i = 0; i < n; ++i) {
    int64_t r, c;
    shape(i, r, c);
    if (!shape_ok(r, c)) return false;
    MatPlan& m = plan.mats[static_cast<size_t>(i)];
    m.rows = r;
    m.cols = c;
    m.colsum_off = plan.colsum_off + static_cast<size_t>(plan.colsum_count) * sizeof(double);
    plan.colsum_count += c;
  }
  off = align_up(plan.colsum_off + static_cast<size_t>(plan.colsum_count) * sizeof(double), kAlign);
  plan.buf_off = off;
  for (int64_t i = 0; i < n; ++i) {
    MatPlan& m = plan.mats[static_cast<size_t>(i)];
    const int64_t r = m.rows, c = m.cols;
    m.tile = tile_class(r, c);
    m.rows_pad = round_up(r, m.tile);
    m.cols_pad = round_up(c, m.tile);
    m.tall = r > c;
    m.m_pad = m.tall ? m.cols_pad : m.rows_pad;
    m.n_pad = m.tall ? m.rows_pad : m.cols_pad;
    m.split = std::min(r, c) <= kSplitMaxM;
    const size_t xb = static_cast<size_t>(m.rows_pad) * static_cast<size_t>(m.cols_pad) * 2;
    const size_t ab = static_cast<size_t>(m.m_pad) * static_cast<size_t>(m.m_pad) * 2;
    m.x_off[0] = off;
    off = align_up(off + xb, kAlign);
    m.x_off[1] = off;
    off = align_up(off + xb, kAlign);
    m.a_off = off;
    off = align_up(off + ab, kAlign);
    m.b_off = off;
    off = align_up(off + ab, kAlign);
    m.blo_off = 0;
    if (m.split) {
      m.blo_off = off;
      off = align_up(off + ab, kAlign);
    }
  }
  plan.total = off;
  return true;
}

// ---------------------------------------------------------------------------
// pinned staging ring for the descriptor upload (per device)
// ---------------------------------------------------------------------------
// Each slot has its own lock: a call waits only for the copy that last used
// the slot it takes (eight calls back), never while holding the library-wide
// lock, so calls on other devices and other slots go on meanwhile.
struct Slot {
  std::mutex mu;
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

constexpr int kSlots = 8;

struct DeviceState {
  Slot slots[kSlots];
  std::atomic<unsigned> next{0};
};

std::mutex g_mu;                       // guards the maps below and the timing record
std::map<int, DeviceState> g_dev;      // node-based: references stay valid

DeviceState& device_state(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  return g_dev[dev];
}

// MUON_DEBUG (environment, read at every call; any value but "" or "0"):
// every launch stays on the caller's stream and is followed by a
// synchronisation and an error check that names the phase, and before a step
// the workspace's iteration buffers (X, A, C of every matrix) are filled with
// bf16 NaN, so that a kernel reading a value that no kernel of the step wrote
// turns the result into NaN.  For debugging only: it serialises the host with
// the device.
thread_local bool g_debug = false;
bool debug_env() {
  const char* v = std::getenv("MUON_DEBUG");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}
constexpr uint32_t kBf16NanPair = 0x7FC07FC0u;

// MUON_CHECK_FINITE (environment, read at every call; any value but "" or
// "0"): at the end of an eager step, wait for the stream and read back the
// squared momentum norms the momentum pass wrote (one double per matrix, slot
// i for the caller's matrix i, zero for a skipped one).  A non-finite norm
// means a NaN or infinite entry in that matrix's new momentum (so in its
// gradient or old momentum), or a sum of squares beyond the fp32 range.
thread_local bool g_check_finite = false;
bool check_finite_env() {
  const char* v = std::getenv("MUON_CHECK_FINITE");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

const char* const kPhaseName[kNumPhases] = {"momentum+norm", "normalise+cast", "Gram X X^T",
                                            "C = aI + bA + cA^2", "X update", "apply",
                                            "AdamW", "fused iteration"};

// timing
struct TimingRec {
  int phase;
  hipEvent_t a, b;
};
bool g_timing = false;
thread_local bool g_no_timing = false;   // set while launching into a capturing stream
std::vector<TimingRec> g_trecs;
std::vector<hipEvent_t> g_evpool;

hipEvent_t pool_event() {
  if (!g_evpool.empty()) {
    hipEvent_t e = g_evpool.back();
    g_evpool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

int hip_fail(hipError_t e, const std::string& what) {
  g_hip_detail = what + ": " + hipGetErrorString(e);
  return MUON_EHIP;
}

// MUON_CHECK_FINITE at the end of a step (see g_check_finite).
int check_norms(const Plan& plan, const char* ws, hipStream_t stream) {
  if (!g_check_finite || plan.n <= 0) return MUON_OK;
  std::vector<double> nrm2(static_cast<size_t>(plan.n));
  hipError_t e = hipMemcpyAsync(nrm2.data(), ws + plan.nrm2_off, nrm2.size() * sizeof(double),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "MUON_CHECK_FINITE read-back of the momentum norms");
  for (size_t i = 0; i < nrm2.size(); ++i) {
    if (!std::isfinite(nrm2[i])) {
      g_hip_detail = "matrix " + std::to_string(i) + ": squared momentum norm is " +
                     (std::isnan(nrm2[i]) ? "NaN" : "infinite");
      return MUON_ENONFINITE;
    }
  }
  return MUON_OK;
}

// False when `stream` belongs to another device than `dev` (a launch there
// would run the library's work on the wrong device).  A stream the runtime
// cannot place (the null stream) is taken as the current device's.
bool stream_on_device(hipStream_t stream, int dev) {
  hipDevice_t sdev = 0;
  if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return true;
  return static_cast<int>(sdev) == dev;
}

int upload_table(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  // the staging ring is reused by later calls: a captured copy would replay
  // whatever the slot holds then
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone) return MUON_ECAPTURE;
  if (!stream_on_device(stream, dev)) return MUON_EINVAL;
  DeviceState& st = device_state(dev);
  Slot& s = st.slots[st.next.fetch_add(1, std::memory_order_relaxed) % kSlots];
  std::lock_guard<std::mutex> lock(s.mu);
  if (s.pending) {
    // wait for the copy that last used this slot (polled: a blocking wait
    // may put the thread to sleep for longer than a small step takes)
    while ((e = hipEventQuery(s.ev)) == hipErrorNotReady) std::this_thread::yield();
    if (e != hipSuccess) return hip_fail(e, "hipEventQuery (staging)");
    s.pending = false;
  }
  if (!s.ev) {
    e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate (staging)");
  }
  if (s.cap < bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(align_up(bytes, 1 << 16), 1 << 16);
    e = hipHostMalloc(&s.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc (staging)");
    s.cap = cap;
  }
  std::memcpy(s.host, src, bytes);
  e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (descriptor table)");
  e = hipEventRecord(s.ev, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord (staging)");
  s.pending = true;
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// side stream: the fused class runs beside the tiled GEMM launches
// ---------------------------------------------------------------------------
// A fork/join pair: a stream (default priority) and the two events that order
// it after the caller's stream and the caller's stream after it again.  The
// eager calls share one pair per device, created on first use and kept for the
// process, and take g_mu around each record + wait so that concurrent callers
// do not reuse an event between the two (a wait takes the event's state at the
// time of the call).  A prepared plan owns a pair of its own, which also joins
// a graph capture of its step.
struct SidePair {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
  bool shared = false;  // the per-device pair: record + wait under g_mu
};
std::map<int, SidePair> g_side;

int make_side(SidePair& sp) {
  hipError_t e = hipStreamCreateWithFlags(&sp.stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&sp.fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&sp.join, hipEventDisableTiming);
  return e == hipSuccess ? MUON_OK : hip_fail(e, "side stream / events");
}

void free_side(SidePair& sp) {
  // work a step queued on the stream runs to completion before its events go
  if (sp.stream) (void)hipStreamSynchronize(sp.stream);
  if (sp.join) (void)hipEventDestroy(sp.join);
  if (sp.fork) (void)hipEventDestroy(sp.fork);
  if (sp.stream) (void)hipStreamDestroy(sp.stream);
  sp = SidePair();
}

// The current device's shared pair.
int shared_side(SidePair*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  SidePair& sp = g_side[dev];
  if (!sp.stream) {
    const int rc = make_side(sp);
    if (rc) {
      free_side(sp);
      return rc;
    }
    sp.shared = true;
  }
  out = &sp;
  return MUON_OK;
}

// `to` waits for everything queued on `from` so far, through `ev`.
int stream_after(const SidePair& sp, hipEvent_t ev, hipStream_t to, hipStream_t from) {
  std::unique_lock<std::mutex> lock(g_mu, std::defer_lock);
  if (sp.shared) lock.lock();
  hipError_t e = hipEventRecord(ev, from);
  if (e == hipSuccess) e = hipStreamWaitEvent(to, ev, 0);
  return e == hipSuccess ? MUON_OK : hip_fail(e, "stream fork / join");
}

// ---------------------------------------------------------------------------
// launch sequence
// ---------------------------------------------------------------------------
template <class F>
int timed(int phase, hipStream_t stream, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  bool timing;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    timing = g_timing && !g_no_timing;
    if (timing) {
      a = pool_event();
      b = pool_event();
      if (!a || !b) return hip_fail(hipErrorOutOfMemory, "hipEventCreate (timing)");
    }
  }
  if (timing) {
    hipError_t e = hipEventRecord(a, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord (timing)");
  }
  const int err = launch();
  if (err != hipSuccess) return hip_fail(static_cast<hipError_t>(err), "kernel launch");
  if (timing) {
    hipError_t e = hipEventRecord(b, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord (timing)");
    std::lock_guard<std::mutex> lock(g_mu);
    g_trecs.push_back({phase, a, b});
  }
  if (g_debug && !g_no_timing) {   // (never while the stream is capturing)
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess)
      return hip_fail(e, std::string("MUON_DEBUG check after the ") + kPhaseName[phase] + " launch");
  }
  return MUON_OK;
}

// MUON_DEBUG: NaN over every matrix's X / A / C buffers before a step.
int debug_poison(const Plan& plan, char* ws, hipStream_t stream) {
  if (!g_debug || g_no_timing || plan.total <= plan.buf_off) return MUON_OK;
  const int err = launch_fill_u32(reinterpret_cast<uint32_t*>(ws + plan.buf_off),
                                  static_cast<int64_t>((plan.total - plan.buf_off) / 4), kBf16NanPair,
                                  static_cast<void*>(stream));
  return err == hipSuccess ? MUON_OK : hip_fail(static_cast<hipError_t>(err), "MUON_DEBUG fill");
}

struct Table {
  std::vector<unsigned char> bytes;
  int n_active = 0;
  int n_big = 0;                      // descriptors [0, n_big): 256-tile matrices,
  int n_small = 0;                    // then n_small 128-tile ones,
  int n_fused = 0;                    // then n_fused fused-kernel ones, by padded
  int fused_n[4] = {};                // short side 32, 64, 96, 128: counts and
  int fused_lds[4] = {};              // largest LDS need per class
  int64_t units[kNumPrefix] = {};
};

bool finite(float x) { return std::isfinite(x); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(int ns_steps, const muon_ns_coeff_t* coeffs, int n_coeffs, float eps) {
  if (ns_steps < 0 || ns_steps > MUON_MAX_NS_STEPS) return MUON_EINVAL;
  if (ns_steps > 0) {
    if (!coeffs || !(n_coeffs == 1 || n_coeffs == ns_steps)) return MUON_EINVAL;
    for (int k = 0; k < n_coeffs; ++k)
      if (!finite(coeffs[k].a) || !finite(coeffs[k].b) || !finite(coeffs[k].c)) return MUON_EINVAL;
  }
  if (!(eps >= 0.0f) || !finite(eps)) return MUON_EINVAL;
  return MUON_OK;
}

// Overlap check over [begin, end) ranges (n log n).
bool any_overlap(std::vector<std::pair<uintptr_t, uintptr_t>>& r) {
  std::sort(r.begin(), r.end());
  for (size_t k = 1; k < r.size(); ++k)
    if (r[k].first < r[k - 1].second) return true;
  return false;
}

// Fill the descriptor table for the active matrices: 256-tile matrices first,
// then 128-tile ones, then the fused class, so each class is one contiguous
// descriptor range.
template <class Fill>
void build_table(const Plan& plan, char* ws, int n_active, Fill fill, Table& t) {
  const size_t n = static_cast<size_t>(plan.n);
  t.bytes.assign(plan.table_bytes, 0);
  t.n_active = n_active;
  MatDesc* desc = reinterpret_cast<MatDesc*>(t.bytes.data() + plan.desc_off);
  int64_t* pre[kNumPrefix];
  for (int k = 0; k < kNumPrefix; ++k)
    pre[k] = reinterpret_cast<int64_t*>(t.bytes.data() + plan.prefix_off[k]);
  int64_t acc[kNumPrefix] = {};
  int a = 0;
  // passes: 256 class, 128 class, then the fused class by padded short side
  for (int pass = 0; pass < 6; ++pass) {
    const int want = pass == 0 ? kTileBig : pass == 1 ? kTileSmall : kTileFused;
    const int fm = kTileFused * (pass - 1);   // fused passes: m_pad 32, 64, 96, 128
    const int sym = pass == 0 ? kPreSymBig : kPreSymSmall;
    const int full = pass == 0 ? kPreFullBig : kPreFullSmall;
    int local = 0;
    for (size_t i = 0; i < n; ++i) {
      const MatPlan& m = plan.mats[i];
      if (m.tile != want || (pass >= 2 && m.m_pad != fm)) continue;
      MatDesc d;
      std::memset(&d, 0, sizeof(d));
      if (!fill(i, d)) continue;
      d.x[0] = reinterpret_cast<uint16_t*>(ws + m.x_off[0]);
      d.x[1] = reinterpret_cast<uint16_t*>(ws + m.x_off[1]);
      d.a = reinterpret_cast<uint16_t*>(ws + m.a_off);
      d.b = reinterpret_cast<uint16_t*>(ws + m.b_off);
      d.blo = m.split ? reinterpret_cast<uint16_t*>(ws + m.blo_off) : nullptr;
      d.nrm2 = reinterpret_cast<double*>(ws + plan.nrm2_off) + i;
      d.rows = m.rows;
      d.cols = m.cols;
      d.rows_pad = static_cast<int32_t>(m.rows_pad);
      d.cols_pad = static_cast<int32_t>(m.cols_pad);
      d.m_pad = static_cast<int32_t>(m.m_pad);
      d.n_pad = static_cast<int32_t>(m.n_pad);
      if (m.tall) d.flags |= kFlagTall;
      if (m.split) d.flags |= kFlagSplitC;
      // row groups of about kChunk elements for the normalise / apply passes
      d.rg_pad = static_cast<int32_t>(std::max<int64_t>(1, kChunk / m.cols_pad));
      d.rg = static_cast<int32_t>(std::max<int64_t>(1, kChunk / m.cols));
      d.colsum = reinterpret_cast<double*>(ws + m.colsum_off);
      d.inv_rows = 1.0 / static_cast<double>(m.rows);
      desc[a] = d;
      const int64_t flat = m.rows * m.cols;
      const int64_t t_side = m.m_pad / m.tile;
      pre[kPreFlat][a] = acc[kPreFlat];
      acc[kPreFlat] += (flat + kChunk - 1) / kChunk;
      pre[kPrePad][a] = acc[kPrePad];
      acc[kPrePad] += (m.rows_pad + d.rg_pad - 1) / d.rg_pad;
      pre[kPreRows][a] = acc[kPreRows];
      acc[kPreRows] += (m.rows + d.rg - 1) / d.rg;
      pre[kPreCol][a] = acc[kPreCol];
      if (d.flags & kFlagZeroCenter)
        acc[kPreCol] += ((m.rows + kColRows - 1) / kColRows) * ((m.cols + kColCols - 1) / kColCols);
      if (pass < 2) {
        pre[sym][local] = acc[sym];
        acc[sym] += t_side * (t_side + 1) / 2;
        pre[full][local] = acc[full];
        acc[full] += (m.rows_pad / m.tile) * (m.cols_pad / m.tile);
      } else {
        int& l = t.fused_lds[pass - 2];
        l = std::max(l, static_cast<int>(fused_lds(m.rows, m.cols)));
      }
      ++a;
      ++local;
    }
    if (pass < 2) {
      pre[sym][local] = acc[sym];
      pre[full][local] = acc[full];
    }
    if (pass == 0) t.n_big = local;
    if (pass == 1) t.n_small = local;
    if (pass >= 2) {
      t.fused_n[pass - 2] = local;
      t.n_fused += local;
    }
  }
  pre[kPreFlat][a] = acc[kPreFlat];
  pre[kPrePad][a] = acc[kPrePad];
  pre[kPreRows][a] = acc[kPreRows];
  pre[kPreCol][a] = acc[kPreCol];
  for (int k = 0; k < kNumPrefix; ++k) t.units[k] = acc[k];
}

// The coefficients travel with the table (the fused kernel reads them).
void fill_coeffs(const Plan& plan, Table& t, int ns_steps, const muon_ns_coeff_t* coeffs,
                 int n_coeffs) {
  float* cf = reinterpret_cast<float*>(t.bytes.data() + plan.coeff_off);
  for (int k = 0; k < (ns_steps > 0 ? n_coeffs : 0); ++k) {
    cf[3 * k] = coeffs[k].a;
    cf[3 * k + 1] = coeffs[k].b;
    cf[3 * k + 2] = coeffs[k].c;
  }
}

// Every launch of one step over a table already in the workspace.  `hyper`
// (device {lr, mu, wd}) overrides the scalar arguments when not null.
// Both a fused class and a tiled class to run: the step forks.
bool wants_side(const Table& t, int ns_steps) {
  return ns_steps > 0 && t.n_fused > 0 && t.n_big + t.n_small > 0;
}

int launch_all(const Plan& plan, const Table& t, char* ws, bool ortho, float lr, float mu,
               float wd, const float* hyper, int ns_steps, const muon_ns_coeff_t* coeffs,
               int n_coeffs, float eps, hipStream_t stream, const SidePair* side) {
  int rc = MUON_OK;
  if (t.n_active == 0) return MUON_OK;
  const MatDesc* d = reinterpret_cast<const MatDesc*>(ws + plan.desc_off);
  const int64_t* pre[kNumPrefix];
  for (int k = 0; k < kNumPrefix; ++k) pre[k] = reinterpret_cast<const int64_t*>(ws + plan.prefix_off[k]);
  const int n = t.n_active, nb = t.n_big, ns = t.n_small, nf = t.n_fused;
  const MatDesc* d_small = d + nb;
  const MatDesc* d_fused = d + nb + ns;
  void* s = static_cast<void*>(stream);
  if (t.units[kPreCol] > 0) {
    // zero-centering: column sums of G first (counted with the momentum phase)
    rc = timed(kPhaseMomentumNorm, stream, [&] {
      return launch_colsum(d, pre[kPreCol], n, t.units[kPreCol],
                           reinterpret_cast<double*>(ws + plan.colsum_off), plan.colsum_count, s);
    });
    if (rc) return rc;
  }
  rc = timed(kPhaseMomentumNorm, stream, [&] {
    return launch_momentum_norm(d, pre[kPreFlat], n, t.units[kPreFlat], mu, hyper, ortho ? 1 : 0, s);
  });
  if (rc) return rc;
  rc = timed(kPhaseNormalize, stream, [&] {
    return launch_normalize(d, pre[kPrePad], n, t.units[kPrePad], eps, mu, hyper, s);
  });
  if (rc) return rc;
  // The fused class and the tiled classes are independent: when both are
  // present the fused launches go to the side stream (forked after the
  // normalisation, joined before the apply pass) and overlap the tiled ones.
  // Phase timing keeps them on one stream, so that each phase's events
  // bracket its own kernels only.
  bool timing;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    timing = g_timing && !g_no_timing;
  }
  const bool fork = side && !timing && !g_debug && nf > 0 && ns_steps > 0 && (nb + ns) > 0;
  hipStream_t fs = fork ? side->stream : stream;
  if (fork) {
    rc = stream_after(*side, side->fork, fs, stream);
    if (rc) return rc;
  }
  const MatDesc* df = d_fused;
  for (int c = 0; c < 4 && nf > 0 && ns_steps > 0; ++c) {
    const int cnt = t.fused_n[c];
    if (cnt == 0) continue;
    rc = timed(kPhaseFusedNS, fs, [&] {
      return launch_ns_fused(kTileFused * (c + 1), df, cnt,
                             reinterpret_cast<const float*>(ws + plan.coeff_off), n_coeffs,
                             ns_steps, t.fused_lds[c], static_cast<void*>(fs));
    });
    if (rc) break;
    df += cnt;
  }
  if (rc) {
    // rejoin even on failure, so that a capture is not left with a loose branch
    if (fork) (void)stream_after(*side, side->join, stream, fs);
    return rc;
  }
  for (int k = 0; k < ((nb + ns) > 0 ? ns_steps : 0); ++k) {
    const muon_ns_coeff_t& c = coeffs[n_coeffs == 1 ? 0 : k];
    const int parity = k & 1;
    rc = timed(kPhaseGram, stream, [&] {
      int e = 0;
      if (nb) e = launch_gram(kTileBig, d, pre[kPreSymBig], nb, t.units[kPreSymBig], parity, s);
      if (!e && ns) e = launch_gram(kTileSmall, d_small, pre[kPreSymSmall], ns, t.units[kPreSymSmall], parity, s);
      return e;
    });
    if (rc) break;
    rc = timed(kPhaseGram2, stream, [&] {
      int e = 0;
      if (nb) e = launch_gram2(kTileBig, d, pre[kPreSymBig], nb, t.units[kPreSymBig], c.a, c.b, c.c, s);
      if (!e && ns) e = launch_gram2(kTileSmall, d_small, pre[kPreSymSmall], ns, t.units[kPreSymSmall], c.a, c.b, c.c, s);
      return e;
    });
    if (rc) break;
    rc = timed(kPhaseXUpdate, stream, [&] {
      int e = 0;
      if (nb) e = launch_xupdate(kTileBig, d, pre[kPreFullBig], nb, t.units[kPreFullBig], parity, s);
      if (!e && ns) e = launch_xupdate(kTileSmall, d_small, pre[kPreFullSmall], ns, t.units[kPreFullSmall], parity, s);
      return e;
    });
    if (rc) break;
  }
  if (fork) {
    const int jrc = stream_after(*side, side->join, stream, fs);
    if (!rc) rc = jrc;
  }
  if (rc) return rc;
  rc = timed(kPhaseApply, stream, [&] {
    return launch_apply(d, pre[kPreRows], n, t.units[kPreRows], ns_steps & 1, lr, wd, mu, hyper,
                        ortho ? 1 : 0, s);
  });
  return rc;
}

int run_sequence(const Plan& plan, Table& t, char* ws, bool ortho, float lr, float mu,
                 float wd, int ns_steps, const muon_ns_coeff_t* coeffs, int n_coeffs, float eps,
                 hipStream_t stream) {
  fill_coeffs(plan, t, ns_steps, coeffs, n_coeffs);
  int rc = upload_table(t.bytes.data(), t.bytes.size(), ws, stream);
  if (rc != MUON_OK) return rc;
  rc = debug_poison(plan, ws, stream);
  if (rc != MUON_OK) return rc;
  SidePair* side = nullptr;
  if (wants_side(t, ns_steps)) {
    rc = shared_side(side);
    if (rc != MUON_OK) return rc;
  }
  return launch_all(plan, t, ws, ortho, lr, mu, wd, nullptr, ns_steps, coeffs, n_coeffs, eps,
                    stream, side);
}

// Validation and descriptor table of a step (muon_step_ex and muon_plan_create).
// Returns MUON_OK with t.n_active == 0 when there is nothing to launch.
int prepare_step(const muon_matrix_t* mats, int64_t n_mats, float lr, float mu, float wd,
                 int ns_steps, const muon_ns_coeff_t* coeffs, int n_coeffs, int rms_scale_mode,
                 float eps, const muon_options_t* options, void* workspace,
                 size_t workspace_bytes, Plan& plan, Table& t) {
  t = Table();
  uint32_t variant = 0;
  if (options) {
    const uint32_t known = MUON_OPT_ZERO_CENTER | MUON_OPT_NESTEROV | MUON_OPT_NS_FIRST;
    if ((options->flags & ~known) != 0 || options->reserved != 0) return MUON_EINVAL;
    if ((options->flags & MUON_OPT_NESTEROV) && (options->flags & MUON_OPT_NS_FIRST)) return MUON_EINVAL;
    if (options->flags & MUON_OPT_ZERO_CENTER) variant |= kFlagZeroCenter;
    if (options->flags & MUON_OPT_NESTEROV) variant |= kFlagNesterov;
    if (options->flags & MUON_OPT_NS_FIRST) variant |= kFlagNsFirst;
  }
  if (n_mats < 0 || (n_mats > 0 && !mats)) return MUON_EINVAL;
  if (n_mats > (int64_t(1) << 24)) return MUON_EINVAL;
  if (!finite(lr) || !finite(mu) || !finite(wd)) return MUON_EINVAL;
  if (rms_scale_mode != MUON_SCALE_NONE && rms_scale_mode != MUON_SCALE_SQRT_MAX1) return MUON_EINVAL;
  int rc = check_common(ns_steps, coeffs, n_coeffs, eps);
  if (rc) return rc;
  if (n_mats == 0) return MUON_OK;
  std::vector<std::pair<uintptr_t, uintptr_t>> ranges;
  int n_active = 0;
  for (int64_t i = 0; i < n_mats; ++i) {
    const muon_matrix_t& m = mats[i];
    if (!shape_ok(m.rows, m.cols)) return MUON_EINVAL;
    if (!m.grad) continue;
    if (!m.param || !m.momentum) return MUON_EINVAL;
    if (m.grad_dtype != MUON_F32 && m.grad_dtype != MUON_BF16) return MUON_EINVAL;
    if (!(m.scale <= 0.0f || finite(m.scale))) return MUON_EINVAL;
    if (std::isnan(m.scale)) return MUON_EINVAL;
    const size_t gsz = m.grad_dtype == MUON_BF16 ? 2 : 4;
    if (!aligned(m.param, 4) || !aligned(m.momentum, 4) || !aligned(m.grad, gsz)) return MUON_EINVAL;
    const size_t el = static_cast<size_t>(m.rows) * static_cast<size_t>(m.cols);
    ranges.push_back({reinterpret_cast<uintptr_t>(m.param), reinterpret_cast<uintptr_t>(m.param) + el * 4});
    ranges.push_back({reinterpret_cast<uintptr_t>(m.momentum), reinterpret_cast<uintptr_t>(m.momentum) + el * 4});
    ranges.push_back({reinterpret_cast<uintptr_t>(m.grad), reinterpret_cast<uintptr_t>(m.grad) + el * gsz});
    ++n_active;
  }
  if (any_overlap(ranges)) return MUON_EALIAS;
  if (!make_plan(n_mats, [&](int64_t i, int64_t& r, int64_t& c) { r = mats[i].rows; c = mats[i].cols; }, plan))
    return MUON_EINVAL;
  if (!workspace || workspace_bytes < plan.total || !aligned(workspace, kAlign)) return MUON_EWORKSPACE;
  if (n_active == 0) return MUON_OK;
  char* ws = static_cast<char*>(workspace);
  build_table(plan, ws, n_active, [&](size_t i, MatDesc& d) {
    const muon_matrix_t& m = mats[i];
    if (!m.grad) return false;
    d.param = m.param;
    d.grad = m.grad;
    d.mom = m.momentum;
    d.flags |= variant;
    const bool bf = m.grad_dtype == MUON_BF16;
    if (bf) d.flags |= kFlagGradBf16;
    const int64_t el = m.rows * m.cols;
    if (el % 8 == 0 && aligned(m.param, 16) && aligned(m.momentum, 16) && aligned(m.grad, 16))
      d.flags |= kFlagVecFlat;
    if ((d.flags & kFlagVecFlat) && m.cols % 8 == 0) d.flags |= kFlagVecRows;
    if (m.scale > 0.0f) d.scale = m.scale;
    else if (rms_scale_mode == MUON_SCALE_SQRT_MAX1)
      d.scale = static_cast<float>(std::sqrt(std::max(1.0, static_cast<double>(m.rows) / static_cast<double>(m.cols))));
    else d.scale = 1.0f;
    return true;
  }, t);
  return MUON_OK;
}

// The last eager step's workspace plan and descriptor table, per thread.  A
// training loop steps the same list every iteration; rebuilding both (argument
// checks, the alias check, the plan, the table) costs about 0.4 ms on the host
// for 2048 matrices, which a step on small matrices does not hide.  The table
// is a pure function of the matrix list, the options, the coefficients and
// the workspace address, all compared byte for byte here, so a hit reuses
// exactly what a rebuild would produce (it is still uploaded every call: the
// workspace's contents are not trusted between calls).
struct StepCache {
  bool valid = false;
  std::vector<muon_matrix_t> mats;
  std::vector<muon_ns_coeff_t> coeffs;
  int ns_steps = 0, n_coeffs = 0, rms_scale_mode = 0;
  uint32_t flags = 0, reserved = 0;
  const void* workspace = nullptr;
  size_t workspace_bytes = 0;
  Plan plan;
  Table t;

  bool matches(const muon_matrix_t* m, int64_t n, int ns, const muon_ns_coeff_t* cf, int nc,
               int rms, const muon_options_t* o, const void* ws, size_t wsb) const {
    if (!valid || n <= 0 || !m || static_cast<size_t>(n) != mats.size() || ns != ns_steps ||
        rms != rms_scale_mode || ws != workspace || wsb != workspace_bytes)
      return false;
    if ((o ? o->flags : 0u) != flags || (o ? o->reserved : 0u) != reserved) return false;
    const int ncf = ns > 0 ? nc : 0;
    if (ncf != static_cast<int>(coeffs.size())) return false;
    if (ncf > 0 && (!cf || std::memcmp(cf, coeffs.data(), sizeof(muon_ns_coeff_t) * ncf) != 0)) return false;
    if (ns > 0 && nc != n_coeffs) return false;
    return std::memcmp(m, mats.data(), sizeof(muon_matrix_t) * mats.size()) == 0;
  }

  void store(const muon_matrix_t* m, int64_t n, int ns, const muon_ns_coeff_t* cf, int nc, int rms,
             const muon_options_t* o, const void* ws, size_t wsb) {
    valid = n > 0 && m != nullptr;
    if (!valid) return;
    mats.assign(m, m + n);
    const int ncf = ns > 0 ? nc : 0;
    coeffs.assign(cf, cf + ncf);
    ns_steps = ns;
    n_coeffs = nc;
    rms_scale_mode = rms;
    flags = o ? o->flags : 0u;
    reserved = o ? o->reserved : 0u;
    workspace = ws;
    workspace_bytes = wsb;
  }
};
thread_local StepCache g_step_cache;

}  // namespace

// A step prepared once over fixed buffers (muon_plan_create).
struct muon_plan {
  Plan plan;
  Table t;
  char* ws = nullptr;
  int device = 0;
  int ns_steps = 0;
  int n_coeffs = 0;
  float eps = 0.f;
  std::vector<muon_ns_coeff_t> coeffs;
  SidePair side;  // own fork / join pair, when the step forks
  ~muon_plan() { free_side(side); }
};

extern "C" {

size_t muon_workspace_bytes(const muon_matrix_t* mats, int64_t n_mats) {
  if (n_mats <= 0 || !mats) return 0;
  Plan plan;
  if (!make_plan(n_mats, [&](int64_t i, int64_t& r, int64_t& c) { r = mats[i].rows; c = mats[i].cols; }, plan))
    return 0;
  return plan.total;
}

int muon_step_ex(const muon_matrix_t* mats, int64_t n_mats, float lr, float mu, float wd,
                 int ns_steps, const muon_ns_coeff_t* coeffs, int n_coeffs, int rms_scale_mode,
                 float eps, const muon_options_t* options, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  g_debug = debug_env();
  g_check_finite = check_finite_env();
  StepCache& c = g_step_cache;
  if (c.matches(mats, n_mats, ns_steps, coeffs, n_coeffs, rms_scale_mode, options, workspace,
                workspace_bytes)) {
    // the list, options and workspace of the last successful call: its plan
    // and table are what a rebuild would produce; only the scalars are new
    if (!finite(lr) || !finite(mu) || !finite(wd) || !(eps >= 0.0f) || !finite(eps)) return MUON_EINVAL;
    if (c.t.n_active == 0) return MUON_OK;
    const int rc = run_sequence(c.plan, c.t, static_cast<char*>(workspace), false, lr, mu, wd,
                                ns_steps, coeffs, n_coeffs, eps, stream);
    return rc != MUON_OK ? rc : check_norms(c.plan, static_cast<const char*>(workspace), stream);
  }
  c.valid = false;
  const int rc = prepare_step(mats, n_mats, lr, mu, wd, ns_steps, coeffs, n_coeffs,
                              rms_scale_mode, eps, options, workspace, workspace_bytes, c.plan, c.t);
  if (rc != MUON_OK) return rc;
  c.store(mats, n_mats, ns_steps, coeffs, n_coeffs, rms_scale_mode, options, workspace,
          workspace_bytes);
  if (c.t.n_active == 0) return MUON_OK;
  const int rc2 = run_sequence(c.plan, c.t, static_cast<char*>(workspace), false, lr, mu, wd,
                               ns_steps, coeffs, n_coeffs, eps, stream);
  return rc2 != MUON_OK ? rc2 : check_norms(c.plan, static_cast<const char*>(workspace), stream);
}

int muon_step(const muon_matrix_t* mats, int64_t n_mats, float lr, float mu, float wd, int ns_steps,
              const muon_ns_coeff_t* coeffs, int n_coeffs, int rms_scale_mode, float eps,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return muon_step_ex(mats, n_mats, lr, mu, wd, ns_steps, coeffs, n_coeffs, rms_scale_mode, eps,
                      nullptr, workspace, workspace_bytes, stream);
}

int muon_step_noalloc(const muon_matrix_t* mats, int64_t n_mats, float lr, float mu, float wd,
                      int ns_steps, const muon_ns_coeff_t* coeffs, int n_coeffs,
                      int rms_scale_mode, float eps, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* ws = nullptr;
  e = static_cast<hipError_t>(noalloc_scratch(dev, &ws));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (scratch)");
  Plan plan;
  Table t;
  // the scratch is checked like a caller's workspace of that size
  int rc = prepare_step(mats, n_mats, lr, mu, wd, ns_steps, coeffs, n_coeffs, rms_scale_mode, eps,
                        nullptr, ws, MUON_NOALLOC_SCRATCH_BYTES, plan, t);
  if (rc != MUON_OK || t.n_active == 0) return rc;
  if (!stream_on_device(stream, dev)) return MUON_EINVAL;
  fill_coeffs(plan, t, ns_steps, coeffs, n_coeffs);
  e = static_cast<hipError_t>(put_bytes(ws, t.bytes.data(), t.bytes.size(), static_cast<void*>(stream)));
  if (e != hipSuccess) return hip_fail(e, "descriptor table (kernel arguments)");
  // no side stream, no timing events, no debug checks: nothing is created
  g_debug = false;
  g_no_timing = true;
  rc = launch_all(plan, t, static_cast<char*>(ws), false, lr, mu, wd, nullptr, ns_steps, coeffs,
                  n_coeffs, eps, stream, nullptr);
  g_no_timing = false;
  return rc;
}

void* muon_noalloc_scratch(void) {
  int dev = 0;
  void* ws = nullptr;
  if (hipGetDevice(&dev) != hipSuccess || noalloc_scratch(dev, &ws) != hipSuccess) return nullptr;
  return ws;
}

int muon_plan_create(const muon_matrix_t* mats, int64_t n_mats, int ns_steps,
                     const muon_ns_coeff_t* coeffs, int n_coeffs, int rms_scale_mode, float eps,
                     const muon_options_t* options, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, muon_plan_t** out) {
  if (!out) return MUON_EINVAL;
  *out = nullptr;
  std::unique_ptr<muon_plan> p(new (std::nothrow) muon_plan());
  if (!p) return hip_fail(hipErrorOutOfMemory, "host allocation of the plan");
  int rc = prepare_step(mats, n_mats, 0.f, 0.f, 0.f, ns_steps, coeffs, n_coeffs, rms_scale_mode,
                        eps, options, workspace, workspace_bytes, p->plan, p->t);
  if (rc != MUON_OK) return rc;
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  p->ws = static_cast<char*>(workspace);
  p->ns_steps = ns_steps;
  p->n_coeffs = n_coeffs;
  p->eps = eps;
  if (ns_steps > 0) p->coeffs.assign(coeffs, coeffs + n_coeffs);
  if (wants_side(p->t, ns_steps)) {
    rc = make_side(p->side);
    if (rc != MUON_OK) return rc;
  }
  if (p->t.n_active > 0) {
    fill_coeffs(p->plan, p->t, ns_steps, coeffs, n_coeffs);
    rc = upload_table(p->t.bytes.data(), p->t.bytes.size(), p->ws, stream);
    if (rc != MUON_OK) return rc;
    e = hipStreamSynchronize(stream);  // the table is in place before the plan is used
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (plan table)");
  }
  *out = p.release();
  return MUON_OK;
}

int muon_plan_step(const muon_plan_t* plan, const float* hyper, hipStream_t stream) {
  if (!plan || !hyper || !aligned(hyper, 4)) return MUON_EINVAL;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device || !stream_on_device(stream, dev)) return MUON_EINVAL;
  if (plan->t.n_active == 0) return MUON_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  // events recorded inside a graph cannot be read back: no phase timing then
  g_no_timing = cap != hipStreamCaptureStatusNone;
  char* ws = plan->ws;
  g_debug = debug_env();
  int rc = debug_poison(plan->plan, ws, stream);
  if (rc == MUON_OK)
    rc = timed(kPhaseMomentumNorm, stream, [&] {
    return launch_fill_zero(reinterpret_cast<double*>(ws + plan->plan.nrm2_off), plan->plan.n,
                            static_cast<void*>(stream));
  });
  if (rc == MUON_OK)
    rc = launch_all(plan->plan, plan->t, ws, false, 0.f, 0.f, 0.f, hyper, plan->ns_steps,
                    plan->coeffs.empty() ? nullptr : plan->coeffs.data(), plan->n_coeffs, plan->eps,
                    stream, plan->side.stream ? &plan->side : nullptr);
  g_no_timing = false;
  // (a capturing stream can neither be waited for nor read back)
  g_check_finite = check_finite_env();
  if (rc == MUON_OK && cap == hipStreamCaptureStatusNone) rc = check_norms(plan->plan, ws, stream);
  return rc;
}

void muon_plan_destroy(muon_plan_t* plan) { delete plan; }

int muon_orthogonalize(const muon_ortho_t* mats, int64_t n_mats, int ns_steps,
                       const muon_ns_coeff_t* coeffs, int n_coeffs, float eps, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  g_debug = debug_env();
  if (n_mats < 0 || (n_mats > 0 && !mats)) return MUON_EINVAL;
  if (n_mats > (int64_t(1) << 24)) return MUON_EINVAL;
  int rc = check_common(ns_steps, coeffs, n_coeffs, eps);
  if (rc) return rc;
  if (n_mats == 0) return MUON_OK;
  std::vector<std::pair<uintptr_t, uintptr_t>> ranges;
  for (int64_t i = 0; i < n_mats; ++i) {
    const muon_ortho_t& m = mats[i];
    if (!shape_ok(m.rows, m.cols)) return MUON_EINVAL;
    if (!m.in || !m.out) return MUON_EINVAL;
    if (m.in_dtype != MUON_F32 && m.in_dtype != MUON_BF16) return MUON_EINVAL;
    const size_t isz = m.in_dtype == MUON_BF16 ? 2 : 4;
    if (!aligned(m.in, isz) || !aligned(m.out, 2)) return MUON_EINVAL;
    const size_t el = static_cast<size_t>(m.rows) * static_cast<size_t>(m.cols);
    ranges.push_back({reinterpret_cast<uintptr_t>(m.out), reinterpret_cast<uintptr_t>(m.out) + el * 2});
    ranges.push_back({reinterpret_cast<uintptr_t>(m.in), reinterpret_cast<uintptr_t>(m.in) + el * isz});
  }
  if (any_overlap(ranges)) return MUON_EALIAS;
  Plan plan;
  if (!make_plan(n_mats, [&](int64_t i, int64_t& r, int64_t& c) { r = mats[i].rows; c = mats[i].cols; }, plan))
    return MUON_EINVAL;
  if (!workspace || workspace_bytes < plan.total || !aligned(workspace, kAlign)) return MUON_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  Table t;
  build_table(plan, ws, static_cast<int>(n_mats), [&](size_t i, MatDesc& d) {
    const muon_ortho_t& m = mats[i];
    d.grad = m.in;
    d.out = static_cast<uint16_t*>(m.out);
    if (m.in_dtype == MUON_BF16) d.flags |= kFlagGradBf16;
    const int64_t el = m.rows * m.cols;
    if (el % 8 == 0 && aligned(m.in, 16) && aligned(m.out, 16)) d.flags |= kFlagVecFlat;
    if ((d.flags & kFlagVecFlat) && m.cols % 8 == 0) d.flags |= kFlagVecRows;
    d.scale = 1.0f;
    return true;
  }, t);
  return run_sequence(plan, t, ws, true, 0.f, 0.f, 0.f, ns_steps, coeffs, n_coeffs, eps, stream);
}

int muon_workspace_view(const muon_matrix_t* mats, int64_t n_mats, int64_t index, int ns_steps,
                        muon_workspace_view_t* view) {
  if (!mats || !view || n_mats <= 0 || index < 0 || index >= n_mats) return MUON_EINVAL;
  if (ns_steps < 0 || ns_steps > MUON_MAX_NS_STEPS) return MUON_EINVAL;
  Plan plan;
  if (!make_plan(n_mats, [&](int64_t i, int64_t& r, int64_t& c) { r = mats[i].rows; c = mats[i].cols; }, plan))
    return MUON_EINVAL;
  const MatPlan& m = plan.mats[static_cast<size_t>(index)];
  view->x_off[0] = m.x_off[0];
  view->x_off[1] = m.x_off[1];
  view->a_off = m.a_off;
  view->c_off = m.b_off;
  view->c_lo_off = m.split ? m.blo_off : 0;
  view->o_off = m.x_off[ns_steps & 1];
  view->nrm2_off = plan.nrm2_off + static_cast<size_t>(index) * sizeof(double);
  view->rows_pad = m.rows_pad;
  view->cols_pad = m.cols_pad;
  view->m_pad = m.m_pad;
  view->transposed = m.tall ? 1 : 0;
  view->tile = m.tile;
  return MUON_OK;
}

// ---------------------------------------------------------------------------
// AdamW branch: [ AdamDesc[n] | prefix int64[n+1] ] in the workspace
// ---------------------------------------------------------------------------
size_t muon_adamw_workspace_bytes(int64_t n_tensors) {
  if (n_tensors <= 0 || n_tensors > (int64_t(1) << 24)) return 0;
  return align_up(static_cast<size_t>(n_tensors) * sizeof(AdamDesc), kAlign) +
         align_up(static_cast<size_t>(n_tensors + 1) * sizeof(int64_t), kAlign);
}

int muon_adamw_step(const muon_adamw_tensor_t* tensors, int64_t n_tensors, float lr, float beta1,
                    float beta2, float eps, float wd, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  g_debug = debug_env();
  if (n_tensors < 0 || (n_tensors > 0 && !tensors)) return MUON_EINVAL;
  if (n_tensors > (int64_t(1) << 24)) return MUON_EINVAL;
  if (!finite(lr) || !finite(wd) || !finite(eps) || !(eps >= 0.0f)) return MUON_EINVAL;
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f)) return MUON_EINVAL;
  if (n_tensors == 0) return MUON_OK;
  std::vector<std::pair<uintptr_t, uintptr_t>> ranges;
  int64_t n_active = 0;
  for (int64_t i = 0; i < n_tensors; ++i) {
    const muon_adamw_tensor_t& t = tensors[i];
    if (t.numel < 1 || t.numel > (int64_t(1) << 40) || t.reserved != 0) return MUON_EINVAL;
    if (!t.grad) continue;
    if (t.step < 1) return MUON_EINVAL;
    if (!t.param || !t.exp_avg || !t.exp_avg_sq) return MUON_EINVAL;
    if (t.grad_dtype != MUON_F32 && t.grad_dtype != MUON_BF16) return MUON_EINVAL;
    const size_t gsz = t.grad_dtype == MUON_BF16 ? 2 : 4;
    if (!aligned(t.param, 4) || !aligned(t.exp_avg, 4) || !aligned(t.exp_avg_sq, 4) || !aligned(t.grad, gsz))
      return MUON_EINVAL;
    const size_t el = static_cast<size_t>(t.numel);
    for (const void* b : {static_cast<const void*>(t.param), static_cast<const void*>(t.exp_avg),
                          static_cast<const void*>(t.exp_avg_sq)})
      ranges.push_back({reinterpret_cast<uintptr_t>(b), reinterpret_cast<uintptr_t>(b) + el * 4});
    ranges.push_back({reinterpret_cast<uintptr_t>(t.grad), reinterpret_cast<uintptr_t>(t.grad) + el * gsz});
    ++n_active;
  }
  if (any_overlap(ranges)) return MUON_EALIAS;
  const size_t need = muon_adamw_workspace_bytes(n_tensors);
  if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)) return MUON_EWORKSPACE;
  if (n_active == 0) return MUON_OK;
  // table: descriptors of the active tensors, then the prefix of their chunk counts
  const size_t desc_bytes = align_up(static_cast<size_t>(n_tensors) * sizeof(AdamDesc), kAlign);
  std::vector<unsigned char> bytes(desc_bytes + static_cast<size_t>(n_active + 1) * sizeof(int64_t), 0);
  AdamDesc* desc = reinterpret_cast<AdamDesc*>(bytes.data());
  int64_t* pre = reinterpret_cast<int64_t*>(bytes.data() + desc_bytes);
  int64_t a = 0, units = 0;
  for (int64_t i = 0; i < n_tensors; ++i) {
    const muon_adamw_tensor_t& t = tensors[i];
    if (!t.grad) continue;
    AdamDesc d;
    std::memset(&d, 0, sizeof(d));
    d.param = t.param;
    d.grad = t.grad;
    d.m = t.exp_avg;
    d.v = t.exp_avg_sq;
    d.numel = t.numel;
    // bias corrections of step t, in double on the host
    const double c1 = 1.0 - std::pow(static_cast<double>(beta1), static_cast<double>(t.step));
    const double c2 = 1.0 - std::pow(static_cast<double>(beta2), static_cast<double>(t.step));
    d.step_size = static_cast<float>(static_cast<double>(lr) / c1);
    d.inv_sqrt_c2 = static_cast<float>(1.0 / std::sqrt(c2));
    d.decay = static_cast<float>(1.0 - static_cast<double>(lr) * static_cast<double>(wd));
    if (t.grad_dtype == MUON_BF16) d.flags |= kFlagGradBf16;
    if (t.numel % 8 == 0 && aligned(t.param, 16) && aligned(t.exp_avg, 16) && aligned(t.exp_avg_sq, 16) &&
        aligned(t.grad, 16))
      d.flags |= kFlagVecFlat;
    desc[a] = d;
    pre[a] = units;
    units += (t.numel + kChunk - 1) / kChunk;
    ++a;
  }
  pre[a] = units;
  char* ws = static_cast<char*>(workspace);
  int rc = upload_table(bytes.data(), bytes.size(), ws, stream);
  if (rc != MUON_OK) return rc;
  const AdamDesc* dd = reinterpret_cast<const AdamDesc*>(ws);
  const int64_t* dp = reinterpret_cast<const int64_t*>(ws + desc_bytes);
  return timed(kPhaseAdamW, stream, [&] {
    return launch_adamw(dd, dp, static_cast<int>(n_active), units, beta1, beta2, eps, static_cast<void*>(stream));
  });
}

int muon_timing_enable(int on) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_timing = on != 0;
  return MUON_OK;
}

int muon_timing_read(double* ms, int64_t* launches) {
  std::vector<TimingRec> recs;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    recs.swap(g_trecs);
  }
  double acc[MUON_PHASES] = {0};
  int64_t cnt[MUON_PHASES] = {0};
  int rc = MUON_OK;
  for (const TimingRec& r : recs) {
    hipError_t e = hipEventSynchronize(r.b);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess && rc == MUON_OK) rc = hip_fail(e, "hipEventElapsedTime");
    if (r.phase >= 0 && r.phase < MUON_PHASES) {
      acc[r.phase] += t;
      cnt[r.phase] += 1;
    }
  }
  {
    std::lock_guard<std::mutex> lock(g_mu);
    for (const TimingRec& r : recs) {
      g_evpool.push_back(r.a);
      g_evpool.push_back(r.b);
    }
  }
  for (int k = 0; k < MUON_PHASES; ++k) {
    if (ms) ms[k] = acc[k];
    if (launches) launches[k] = cnt[k];
  }
  return rc;
}

const char* muon_status_string(int status) {
  static thread_local std::string s;
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_EINVAL: return "invalid argument";
    case MUON_EWORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case MUON_EALIAS: return "param / grad / momentum (or in / out) ranges overlap";
    case MUON_ECAPTURE:
      return "the stream is capturing a graph: calls stage their descriptor table through "
             "reused host buffers and cannot be captured";
    case MUON_EHIP:
      s = "HIP error: " + g_hip_detail;
      return s.c_str();
    case MUON_ENONFINITE:
      s = "non-finite values (MUON_CHECK_FINITE): " + g_hip_detail;
      return s.c_str();
    default: return "unknown status";
  }
}

const char* muon_version(void) { return "libmuon 0.1 gfx950"; }

}  // extern "C"
