// Host-side replay of libmuon's dispatcher (muon_api.cpp, compiled unchanged
// with the host C++ compiler) on the CPU: the HIP runtime calls it makes are
// replaced by plain host stand-ins (a "device" buffer is host memory, a copy
// is memcpy, streams and events are inert), and every kernel launcher records
// its arguments instead of launching.  The checks then read the descriptor
// table and prefix arrays the dispatcher really built, exactly as a kernel
// would find them in the workspace:
//   * the launch sequence: one launch per phase, the Gram / C / X-update
//     triple per Newton-Schulz step and tile class, in order; the apply pass
//     reads the iterate of parity ns_steps & 1; each C launch gets its step's
//     coefficients;
//   * each launch's unit count equals its prefix array's total, and each
//     matrix owns t (t + 1) / 2 upper tiles (symmetric phases) or every tile
//     (X update), with t = m_pad / tile;
//   * every descriptor's workspace buffers (X0, X1, A, C, C_lo, norm slot,
//     column sums) lie inside the workspace, 256-byte aligned where they are
//     operands, sized for the padded shape, and disjoint across matrices;
//     padding, orientation, split-C and vectorisation flags follow the shape;
//     skipped matrices (no gradient) have no descriptor.
// Usage: host_replay <case>; prints "ok" and exits 0, or the first failure.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "muon.h"
#include "muon_internal.h"

// ---------------------------------------------------------------- HIP ----
extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
  *s = hipStreamCaptureStatusNone;
  return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) { *d = 0; return hipSuccess; }
hipError_t hipEventQuery(hipEvent_t) { return hipSuccess; }
hipError_t hipEventCreate(hipEvent_t* e) { *e = reinterpret_cast<hipEvent_t>(new int(0)); return hipSuccess; }
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) { delete reinterpret_cast<int*>(e); return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0.f; return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "replay"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) {
  *p = std::malloc(n);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostFree(void* p) { std::free(p); return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned) {
  *s = reinterpret_cast<hipStream_t>(new int(0));
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) { delete reinterpret_cast<int*>(s); return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
}

// ---------------------------------------------------------- launchers ----
namespace muon {
struct Launch {
  std::string phase;
  int tile = 0;
  const MatDesc* d = nullptr;
  const int64_t* prefix = nullptr;
  int n = 0;
  int64_t units = 0;
  int parity = -1;
  float a = 0, b = 0, c = 0;
};
std::vector<Launch> g_log;

static int rec(const char* phase, int tile, const MatDesc* d, const int64_t* prefix, int n,
               int64_t units, int parity = -1, float a = 0, float b = 0, float c = 0) {
  Launch l;
  l.phase = phase; l.tile = tile; l.d = d; l.prefix = prefix; l.n = n; l.units = units;
  l.parity = parity; l.a = a; l.b = b; l.c = c;
  g_log.push_back(l);
  return 0;
}
// The momentum stand-in can leave a chosen value in one descriptor's norm
// slot, as the momentum pass does for a matrix with a non-finite entry.
int g_plant_desc = -1;
double g_plant_value = 0.0;
double* g_planted_slot = nullptr;
int launch_momentum_norm(const MatDesc* d, const int64_t* p, int n, int64_t u, float, const float*, int, void*) {
  if (g_plant_desc >= 0 && g_plant_desc < n) {
    g_planted_slot = d[g_plant_desc].nrm2;
    *g_planted_slot = g_plant_value;
  }
  return rec("momentum", 0, d, p, n, u);
}
int launch_normalize(const MatDesc* d, const int64_t* p, int n, int64_t u, float, float, const float*, void*) {
  return rec("normalize", 0, d, p, n, u);
}
int launch_fill_zero(double*, int64_t, void*) { return rec("fill", 0, nullptr, nullptr, 0, 0); }
int launch_fill_u32(uint32_t*, int64_t, uint32_t, void*) { return rec("poison", 0, nullptr, nullptr, 0, 0); }
int launch_colsum(const MatDesc* d, const int64_t* p, int n, int64_t u, double*, int64_t, void*) {
  return rec("colsum", 0, d, p, n, u);
}
int launch_gram(int tile, const MatDesc* d, const int64_t* p, int n, int64_t u, int parity, void*) {
  return rec("gram", tile, d, p, n, u, parity);
}
int launch_gram2(int tile, const MatDesc* d, const int64_t* p, int n, int64_t u, float a, float b, float c, void*) {
  return rec("gram2", tile, d, p, n, u, -1, a, b, c);
}
int launch_xupdate(int tile, const MatDesc* d, const int64_t* p, int n, int64_t u, int parity, void*) {
  return rec("xupdate", tile, d, p, n, u, parity);
}
int launch_apply(const MatDesc* d, const int64_t* p, int n, int64_t u, int parity, float, float, float,
                 const float*, int, void*) {
  return rec("apply", 0, d, p, n, u, parity);
}
int launch_adamw(const AdamDesc*, const int64_t*, int, int64_t, float, float, float, void*) {
  return rec("adamw", 0, nullptr, nullptr, 0, 0);
}
int launch_ns_fused(int m_pad, const MatDesc* d, int n, const float*, int, int, int, void*) {
  return rec("fused", m_pad, d, nullptr, n, n);
}
int noalloc_scratch(int, void**) { return static_cast<int>(hipErrorNotSupported); }
int put_bytes(void*, const void*, size_t, void*) { return static_cast<int>(hipErrorNotSupported); }
}  // namespace muon

// ------------------------------------------------------------- checks ----
using namespace muon;
static int g_fail = 0;
#define CHECK(cond, ...)                                     \
  do {                                                       \
    if (!(cond)) {                                           \
      if (g_fail++ < 10) {                                   \
        std::printf("FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
        std::printf(__VA_ARGS__);                            \
        std::printf("\n");                                   \
      }                                                      \
    }                                                        \
  } while (0)

static int64_t ceil_to(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

enum Entry { kEager = 0, kPlan = 1, kOrtho = 2 };
struct Case {
  std::vector<std::pair<int64_t, int64_t>> shapes;
  std::vector<bool> present;
  int ns = 5;
  std::vector<muon_ns_coeff_t> coeffs{{3.4445f, -4.7750f, 2.0315f}};
  uint32_t opts = 0;       // MUON_OPT_* of muon_step_ex (eager and plan)
  int entry = kEager;
  int rms = MUON_SCALE_NONE;
};

static void check_call(const char* name, const Case& cs, std::vector<muon_matrix_t>& mats, char* ws,
                       size_t ws_bytes);

static void run_case(const char* name, const Case& cs) {
  const int64_t n = static_cast<int64_t>(cs.shapes.size());
  std::vector<muon_matrix_t> mats(n);
  for (int64_t i = 0; i < n; ++i) {
    muon_matrix_t& m = mats[i];
    m.rows = cs.shapes[i].first;
    m.cols = cs.shapes[i].second;
    m.grad_dtype = MUON_BF16;
    m.scale = 0.f;
    // caller buffers: distinct, 16-byte aligned addresses (never dereferenced)
    const uintptr_t base = 0x100000000000ull + static_cast<uintptr_t>(i) * 0x100000000ull;
    m.param = reinterpret_cast<float*>(base);
    m.momentum = reinterpret_cast<float*>(base + 0x40000000ull);
    m.grad = cs.present.empty() || cs.present[i] ? reinterpret_cast<void*>(base + 0x80000000ull) : nullptr;
  }
  const size_t ws_bytes = muon_workspace_bytes(mats.data(), n);
  CHECK(ws_bytes > 0, "%s: workspace size", name);
  // the workspace: host memory standing in for device memory (untouched pages stay virtual)
  char* raw = static_cast<char*>(std::malloc(ws_bytes + 256));
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(raw) + 255) & ~uintptr_t(255));
  // the same list twice (the second eager call reuses the first one's plan
  // and table), then with the first matrix's gradient toggled (rebuilt)
  check_call(name, cs, mats, ws, ws_bytes);
  if (cs.entry != kEager) {
    std::free(raw);
    return;
  }
  std::memset(ws, 0xA5, std::min<size_t>(ws_bytes, 1 << 22));   // the table is uploaded anew
  check_call(name, cs, mats, ws, ws_bytes);
  Case cs2 = cs;
  if (cs2.present.empty()) cs2.present.assign(static_cast<size_t>(n), true);
  cs2.present[0] = !cs2.present[0];
  mats[0].grad = cs2.present[0] ? reinterpret_cast<void*>(0x100000000000ull + 0x80000000ull) : nullptr;
  check_call(name, cs2, mats, ws, ws_bytes);
  std::free(raw);
}

static void check_call(const char* name, const Case& cs, std::vector<muon_matrix_t>& mats, char* ws,
                       size_t ws_bytes) {
  const int64_t n_all = static_cast<int64_t>(mats.size());
  g_log.clear();
  const muon_options_t opt{cs.opts, 0u};
  int rc = MUON_OK;
  std::vector<muon_ortho_t> orth;
  if (cs.entry == kEager) {
    rc = muon_step_ex(mats.data(), n_all, 0.02f, 0.95f, 0.01f, cs.ns, cs.coeffs.data(),
                      static_cast<int>(cs.coeffs.size()), cs.rms, 1e-7f, &opt, ws, ws_bytes, nullptr);
  } else if (cs.entry == kPlan) {
    muon_plan_t* plan = nullptr;
    rc = muon_plan_create(mats.data(), n_all, cs.ns, cs.coeffs.data(), static_cast<int>(cs.coeffs.size()),
                          cs.rms, 1e-7f, &opt, ws, ws_bytes, nullptr, &plan);
    CHECK(g_log.empty(), "%s: plan creation launched kernels", name);
    const float hyper[3] = {0.02f, 0.95f, 0.01f};          // "device" floats
    if (rc == MUON_OK) rc = muon_plan_step(plan, hyper, nullptr);
    muon_plan_destroy(plan);
    // a plan step first clears the norm slots with a fill kernel
    CHECK(!g_log.empty() && g_log.front().phase == "fill", "%s: plan step without its fill", name);
    if (!g_log.empty()) g_log.erase(g_log.begin());
  } else {
    // orthogonalisation alone: in = the gradient, out = a bf16 buffer at the parameter's address;
    // skipped matrices are left out of the list
    std::vector<muon_matrix_t> kept;
    for (const muon_matrix_t& m : mats)
      if (m.grad) {
        muon_ortho_t o;
        o.in = m.grad;
        o.out = m.param;
        o.rows = m.rows;
        o.cols = m.cols;
        o.in_dtype = m.grad_dtype;
        orth.push_back(o);
        kept.push_back(m);
      }
    mats = kept;
    rc = orth.empty() ? MUON_OK
                      : muon_orthogonalize(orth.data(), static_cast<int64_t>(orth.size()), cs.ns,
                                           cs.coeffs.data(), static_cast<int>(cs.coeffs.size()), 1e-7f,
                                           ws, ws_bytes, nullptr);
  }
  CHECK(rc == MUON_OK, "%s: entry %d returned %d", name, cs.entry, rc);
  if (rc != MUON_OK) return;
  const int64_t n = static_cast<int64_t>(mats.size());      // (orthogonalise: the present ones)
  if (mats.empty() || g_log.empty()) {
    CHECK(g_log.empty(), "%s: launches for an empty list", name);
    return;
  }

  // expected classes, from the shapes alone (the kernels' class rules)
  auto fused = [](int64_t r, int64_t c) {
    const int64_t m = ceil_to(std::min(r, c), kTileFused), nn = ceil_to(std::max(r, c), kTileFused);
    return m <= kFusedMaxM && 2 * (m * ceil_to(nn, 128) + 2 * m * ceil_to(m, 128)) <= kFusedLdsMax;
  };
  auto tile_of = [&](int64_t r, int64_t c) {
    return std::min(r, c) >= kBigMinM ? kTileBig : (fused(r, c) ? kTileFused : kTileSmall);
  };
  int n_active = 0, n_big = 0, n_small = 0, n_fused = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (!mats[i].grad) continue;
    ++n_active;
    const int t = tile_of(mats[i].rows, mats[i].cols);
    (t == kTileBig ? n_big : t == kTileSmall ? n_small : n_fused) += 1;
  }

  if (n_active == 0) {
    CHECK(g_log.empty(), "%s: launches with every gradient absent", name);
    return;
  }
  // the launch sequence
  std::vector<std::string> want;
  if (cs.opts & MUON_OPT_ZERO_CENTER) want.push_back("colsum");
  want.push_back("momentum");
  want.push_back("normalize");
  int fused_launches = 0;
  for (const Launch& l : g_log) fused_launches += l.phase == "fused";
  {
    // one fused launch per padded short side present (when there is an iteration)
    bool seen[5] = {false, false, false, false, false};
    int classes = 0;
    for (int64_t i = 0; i < n; ++i)
      if (mats[i].grad && tile_of(mats[i].rows, mats[i].cols) == kTileFused) {
        const int k = static_cast<int>(ceil_to(std::min(mats[i].rows, mats[i].cols), kTileFused) / kTileFused);
        if (!seen[k]) classes += 1;
        seen[k] = true;
      }
    CHECK(fused_launches == (cs.ns > 0 ? classes : 0), "%s: %d fused launches, want %d", name,
          fused_launches, cs.ns > 0 ? classes : 0);
  }
  for (int f = 0; f < fused_launches; ++f) want.push_back("fused");
  for (int k = 0; k < ((n_big + n_small) ? cs.ns : 0); ++k)
    for (const char* ph : {"gram", "gram2", "xupdate"}) {
      if (n_big) want.push_back(ph);
      if (n_small) want.push_back(ph);
    }
  want.push_back("apply");
  CHECK(g_log.size() == want.size(), "%s: %zu launches, want %zu", name, g_log.size(), want.size());
  for (size_t k = 0; k < std::min(g_log.size(), want.size()); ++k)
    CHECK(g_log[k].phase == want[k], "%s: launch %zu is %s, want %s", name, k, g_log[k].phase.c_str(),
          want[k].c_str());
  CHECK(!(n_fused && !fused_launches && cs.ns > 0), "%s: fused matrices but no fused launch", name);

  // descriptors, read from the table the dispatcher uploaded into the workspace
  const MatDesc* d = g_log.front().d;
  CHECK(reinterpret_cast<const char*>(d) == ws, "%s: descriptor table at the workspace base", name);
  CHECK(g_log.front().n == n_active, "%s: %d descriptors, want %d", name, g_log.front().n, n_active);
  std::vector<std::pair<uintptr_t, uintptr_t>> regions;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ws), hi = lo + ws_bytes;
  auto inside = [&](const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return a >= lo && a + bytes <= hi;
  };
  for (int a = 0; a < n_active; ++a) {
    const MatDesc& m = d[a];
    // class order: 256-tiles, 128-tiles, then the fused class
    const int t = tile_of(m.rows, m.cols);
    const int cls = t == kTileBig ? 0 : t == kTileSmall ? 1 : 2;
    const int want_cls = a < n_big ? 0 : a < n_big + n_small ? 1 : 2;
    CHECK(cls == want_cls, "%s: descriptor %d in class %d, want %d", name, a, cls, want_cls);
    const int64_t rp = ceil_to(m.rows, t), cp = ceil_to(m.cols, t);
    const bool tall = m.rows > m.cols;
    CHECK(m.rows_pad == rp && m.cols_pad == cp, "%s: descriptor %d padding", name, a);
    CHECK(m.m_pad == (tall ? cp : rp) && m.n_pad == (tall ? rp : cp), "%s: descriptor %d m/n pad", name, a);
    CHECK(((m.flags & kFlagTall) != 0) == tall, "%s: descriptor %d tall flag", name, a);
    CHECK(((m.flags & kFlagSplitC) != 0) == (std::min(m.rows, m.cols) <= kSplitMaxM),
          "%s: descriptor %d split flag", name, a);
    CHECK((m.flags & kFlagGradBf16) != 0, "%s: descriptor %d dtype", name, a);
    const size_t xb = static_cast<size_t>(rp) * cp * 2, ab = static_cast<size_t>(m.m_pad) * m.m_pad * 2;
    for (int k = 0; k < 2; ++k) {
      CHECK(inside(m.x[k], xb) && reinterpret_cast<uintptr_t>(m.x[k]) % 256 == 0, "%s: X%d of %d", name, k, a);
      regions.push_back({reinterpret_cast<uintptr_t>(m.x[k]), reinterpret_cast<uintptr_t>(m.x[k]) + xb});
    }
    for (const uint16_t* p : {m.a, m.b}) {
      CHECK(inside(p, ab) && reinterpret_cast<uintptr_t>(p) % 256 == 0, "%s: A/C of %d", name, a);
      regions.push_back({reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + ab});
    }
    if (m.flags & kFlagSplitC) {
      CHECK(m.blo && inside(m.blo, ab), "%s: C_lo of %d", name, a);
      regions.push_back({reinterpret_cast<uintptr_t>(m.blo), reinterpret_cast<uintptr_t>(m.blo) + ab});
    } else {
      CHECK(m.blo == nullptr, "%s: C_lo of unsplit %d", name, a);
    }
    CHECK(inside(m.nrm2, 8), "%s: norm slot of %d", name, a);
    regions.push_back({reinterpret_cast<uintptr_t>(m.nrm2), reinterpret_cast<uintptr_t>(m.nrm2) + 8});
    CHECK(inside(m.colsum, static_cast<size_t>(m.cols) * 8), "%s: column sums of %d", name, a);
    regions.push_back({reinterpret_cast<uintptr_t>(m.colsum),
                       reinterpret_cast<uintptr_t>(m.colsum) + static_cast<size_t>(m.cols) * 8});
  }
  std::sort(regions.begin(), regions.end());
  for (size_t k = 1; k < regions.size(); ++k)
    CHECK(regions[k].first >= regions[k - 1].second, "%s: workspace regions overlap", name);
  // every active matrix's caller pointers appear exactly once (orthogonalisation:
  // its input and output), and the step variants travel in the flags
  std::vector<const void*> grads;
  for (int a = 0; a < n_active; ++a) {
    grads.push_back(d[a].grad);
    if (cs.entry == kOrtho) {
      CHECK(d[a].param == nullptr && d[a].mom == nullptr && d[a].out != nullptr, "%s: ortho descriptor %d", name, a);
    } else {
      CHECK(d[a].out == nullptr && d[a].param != nullptr && d[a].mom != nullptr, "%s: step descriptor %d", name, a);
      const uint32_t want_flags = ((cs.opts & MUON_OPT_ZERO_CENTER) ? kFlagZeroCenter : 0u) |
                                  ((cs.opts & MUON_OPT_NESTEROV) ? kFlagNesterov : 0u) |
                                  ((cs.opts & MUON_OPT_NS_FIRST) ? kFlagNsFirst : 0u);
      CHECK((d[a].flags & (kFlagZeroCenter | kFlagNesterov | kFlagNsFirst)) == want_flags,
            "%s: variant flags of %d", name, a);
    }
    const double want_scale = cs.rms == MUON_SCALE_SQRT_MAX1
                                  ? std::sqrt(std::max(1.0, double(d[a].rows) / double(d[a].cols)))
                                  : 1.0;
    CHECK(cs.entry == kOrtho || std::fabs(d[a].scale - want_scale) <= 1e-6 * want_scale,
          "%s: scale of %d", name, a);
  }
  std::sort(grads.begin(), grads.end());
  CHECK(std::adjacent_find(grads.begin(), grads.end()) == grads.end(), "%s: a gradient twice", name);
  for (int64_t i = 0; i < n; ++i)
    CHECK(std::binary_search(grads.begin(), grads.end(), static_cast<const void*>(mats[i].grad)) ==
              (mats[i].grad != nullptr),
          "%s: matrix %lld presence", name, static_cast<long long>(i));

  // per-launch units against the prefix arrays and the tile counts
  int step_of_gram2 = 0;
  for (const Launch& l : g_log) {
    if (l.phase == "gram" || l.phase == "gram2" || l.phase == "xupdate") {
      const bool sym = l.phase != "xupdate";
      CHECK(l.prefix[0] == 0 && l.prefix[l.n] == l.units, "%s: %s units %lld, prefix total %lld", name,
            l.phase.c_str(), static_cast<long long>(l.units), static_cast<long long>(l.prefix[l.n]));
      for (int i = 0; i < l.n; ++i) {
        const MatDesc& m = l.d[i];
        CHECK(m.m_pad % l.tile == 0 && m.n_pad % l.tile == 0, "%s: %s tile %d", name, l.phase.c_str(), l.tile);
        const int64_t ts = m.m_pad / l.tile;
        const int64_t own = sym ? ts * (ts + 1) / 2 : (m.rows_pad / l.tile) * (m.cols_pad / l.tile);
        CHECK(l.prefix[i + 1] - l.prefix[i] == own, "%s: %s matrix %d owns %lld units, want %lld", name,
              l.phase.c_str(), i, static_cast<long long>(l.prefix[i + 1] - l.prefix[i]),
              static_cast<long long>(own));
      }
      if (l.phase == "gram2") {
        const muon_ns_coeff_t& c = cs.coeffs[cs.coeffs.size() == 1 ? 0 : step_of_gram2 / ((n_big > 0) + (n_small > 0))];
        CHECK(l.a == c.a && l.b == c.b && l.c == c.c, "%s: C launch coefficients", name);
        ++step_of_gram2;
      }
    }
    if (l.phase == "apply") CHECK(l.parity == (cs.ns & 1), "%s: apply parity %d", name, l.parity);
  }
}

// MUON_CHECK_FINITE: a step reads back the momentum norms and reports the
// first non-finite one by the caller's matrix index, on the eager path (first
// call and the cached repeat) and on a plan step; without the variable the
// same planted value passes unnoticed.
static void finite_check(const Case& cs) {
  const int64_t n = static_cast<int64_t>(cs.shapes.size());
  std::vector<muon_matrix_t> mats(n);
  for (int64_t i = 0; i < n; ++i) {
    muon_matrix_t& m = mats[i];
    m.rows = cs.shapes[i].first;
    m.cols = cs.shapes[i].second;
    m.grad_dtype = MUON_BF16;
    m.scale = 0.f;
    const uintptr_t base = 0x100000000000ull + static_cast<uintptr_t>(i) * 0x100000000ull;
    m.param = reinterpret_cast<float*>(base);
    m.momentum = reinterpret_cast<float*>(base + 0x40000000ull);
    m.grad = cs.present.empty() || cs.present[i] ? reinterpret_cast<void*>(base + 0x80000000ull) : nullptr;
  }
  const size_t ws_bytes = muon_workspace_bytes(mats.data(), n);
  char* raw = static_cast<char*>(std::malloc(ws_bytes + 256));
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(raw) + 255) & ~uintptr_t(255));
  const int nc = static_cast<int>(cs.coeffs.size());
  auto step = [&]() {
    return muon_step(mats.data(), n, 0.02f, 0.95f, 0.01f, cs.ns, cs.coeffs.data(), nc, cs.rms, 1e-7f,
                     ws, ws_bytes, nullptr);
  };
  // the caller's index of the planted slot
  auto planted_index = [&]() -> int64_t {
    for (int64_t i = 0; i < n; ++i) {
      muon_workspace_view_t v;
      if (muon_workspace_view(mats.data(), n, i, cs.ns, &v) == MUON_OK &&
          reinterpret_cast<double*>(ws + v.nrm2_off) == g_planted_slot)
        return i;
    }
    return -1;
  };
  unsetenv("MUON_CHECK_FINITE");
  g_plant_desc = 0;
  g_plant_value = std::nan("");
  CHECK(step() == MUON_OK, "finite: unchecked step with a NaN norm");
  setenv("MUON_CHECK_FINITE", "1", 1);
  g_plant_desc = -1;
  CHECK(step() == MUON_OK, "finite: checked step, all finite");
  int n_active = 0;
  for (const auto& l : g_log)
    if (l.phase == "momentum") n_active = l.n;
  CHECK(n_active > 2, "finite: %d active descriptors", n_active);
  const int picks[3] = {0, n_active / 2, n_active - 1};
  for (int k : picks) {
    for (int kind = 0; kind < 2; ++kind) {
      g_plant_desc = k;
      g_plant_value = kind == 0 ? std::nan("") : HUGE_VAL;
      for (int rep = 0; rep < 2; ++rep) {            // the first call and the cached repeat
        g_log.clear();
        const int rc = step();
        const int64_t want = planted_index();
        CHECK(want >= 0 && (cs.present.empty() || cs.present[static_cast<size_t>(want)]),
              "finite: planted slot %d maps to no active matrix", k);
        CHECK(rc == MUON_ENONFINITE, "finite: descriptor %d kind %d rep %d gave %d", k, kind, rep, rc);
        const std::string msg = muon_status_string(rc);
        const std::string tag = "matrix " + std::to_string(want) + ":";
        CHECK(msg.find(tag) != std::string::npos && msg.find(kind == 0 ? "NaN" : "infinite") != std::string::npos,
              "finite: status '%s' does not name %s", msg.c_str(), tag.c_str());
      }
    }
  }
  // a plan step checks too
  g_plant_desc = n_active - 1;
  g_plant_value = std::nan("");
  muon_plan_t* plan = nullptr;
  int rc = muon_plan_create(mats.data(), n, cs.ns, cs.coeffs.data(), nc, cs.rms, 1e-7f, nullptr, ws,
                            ws_bytes, nullptr, &plan);
  CHECK(rc == MUON_OK, "finite: plan create %d", rc);
  const float hyper[3] = {0.02f, 0.95f, 0.01f};
  if (rc == MUON_OK) {
    rc = muon_plan_step(plan, hyper, nullptr);
    CHECK(rc == MUON_ENONFINITE, "finite: plan step gave %d", rc);
    muon_plan_destroy(plan);
  }
  unsetenv("MUON_CHECK_FINITE");
  g_plant_desc = -1;
  std::free(raw);
}

int main(int argc, char** argv) {
  const std::string which = argc > 1 ? argv[1] : "all";
  Case mamba;
  for (int l = 0; l < 24; ++l)
    for (auto s : {std::make_pair(768, 3072), std::make_pair(1536, 80), std::make_pair(48, 1536),
                   std::make_pair(1536, 768)})
      mamba.shapes.push_back(s);
  Case transformer;  // 8 of the 32 layers (the workspace is host memory here)
  for (int l = 0; l < 8; ++l) {
    for (int k = 0; k < 4; ++k) transformer.shapes.push_back({4096, 4096});
    transformer.shapes.push_back({4096, 14336});
    transformer.shapes.push_back({4096, 14336});
    transformer.shapes.push_back({14336, 4096});
  }
  Case ragged;
  unsigned x = 12345u;
  const int64_t sz[4] = {64, 128, 256, 512};
  for (int i = 0; i < 2048; ++i) {
    x = x * 1664525u + 1013904223u;
    const int64_t r = sz[(x >> 10) & 3];
    x = x * 1664525u + 1013904223u;
    ragged.shapes.push_back({r, sz[(x >> 10) & 3]});
  }
  Case mixed;  // every class, both orientations, ragged edges, skipped matrices, per-step coefficients
  mixed.shapes = {{20, 300}, {300, 50}, {96, 200}, {128, 384}, {48, 1536}, {1536, 80}, {130, 700},
                  {700, 300}, {200, 200}, {1030, 1280}, {1280, 1030}, {1, 1}, {8192, 28672}, {33, 7}};
  mixed.present = {true, true, false, true, true, true, true, false, true, true, true, true, true, true};
  mixed.ns = 10;
  mixed.coeffs.clear();
  for (int k = 0; k < 10; ++k)
    mixed.coeffs.push_back(k < 8 ? muon_ns_coeff_t{3.4445f, -4.7750f, 2.0315f} : muon_ns_coeff_t{2.f, -1.5f, 0.5f});
  if (which == "random") {
    // a seeded random list: shapes across every kernel class and both
    // orientations (sides 1..4000, mostly small), a tenth of the gradients
    // absent, 0..12 Newton-Schulz steps with one or per-step coefficients,
    // any accepted variant combination, RMS scale on or off, and the eager,
    // plan or orthogonalise entry
    const unsigned seed = argc > 2 ? static_cast<unsigned>(std::atoi(argv[2])) : 1u;
    unsigned r = seed * 2654435761u + 12345u;
    auto next = [&r](unsigned mod) {
      r = r * 1664525u + 1013904223u;
      return (r >> 8) % mod;
    };
    auto side = [&]() -> int64_t {
      const unsigned k = next(100);
      if (k < 35) return 1 + next(32);
      if (k < 65) return 33 + next(96);
      if (k < 93) return 129 + next(900);
      return 1000 + next(3000);
    };
    Case rc;
    const int n = 1 + static_cast<int>(next(160));
    for (int i = 0; i < n; ++i) {
      rc.shapes.push_back({side(), side()});
      rc.present.push_back(next(10) != 0);
    }
    rc.ns = static_cast<int>(next(13));
    rc.coeffs.clear();
    const int nc = (next(2) == 0 || rc.ns == 0) ? 1 : rc.ns;
    for (int k = 0; k < nc; ++k)
      rc.coeffs.push_back({1.0f + 0.25f * next(10), -0.5f - 0.25f * next(16), 0.1f * next(25)});
    const uint32_t combos[6] = {0u, MUON_OPT_ZERO_CENTER, MUON_OPT_NESTEROV, MUON_OPT_NS_FIRST,
                                MUON_OPT_ZERO_CENTER | MUON_OPT_NESTEROV,
                                MUON_OPT_ZERO_CENTER | MUON_OPT_NS_FIRST};
    rc.entry = static_cast<int>(next(3));
    rc.opts = rc.entry == kOrtho ? 0u : combos[next(6)];
    rc.rms = next(2) ? MUON_SCALE_SQRT_MAX1 : MUON_SCALE_NONE;
    const std::string nm = "random " + std::to_string(seed);
    run_case(nm.c_str(), rc);
  }
  if (which == "all" || which == "finite") finite_check(mixed);
  if (which == "all" || which == "mamba") run_case("mamba", mamba);
  if (which == "all" || which == "transformer") run_case("transformer", transformer);
  if (which == "all" || which == "ragged") run_case("ragged", ragged);
  if (which == "all" || which == "mixed") run_case("mixed", mixed);
  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}
