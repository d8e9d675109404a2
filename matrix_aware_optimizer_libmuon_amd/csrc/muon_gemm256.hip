// Tile-256 instantiation of the Newton-Schulz GEMM kernels (muon_gemm.h).
// Built with MFMA accumulators in the accumulator registers (256 of them).
#include "muon_gemm.h"

namespace muon {

int launch_gram_256(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                   void* stream) {
  return launch_gram_t<256>(d, prefix, n, units, parity, stream);
}

int launch_gram2_256(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a,
                    float b, float c, void* stream) {
  return launch_gram2_t<256>(d, prefix, n, units, a, b, c, stream);
}

int launch_xupdate_256(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                      void* stream) {
  return launch_xupdate_t<256>(d, prefix, n, units, parity, stream);
}

}  // namespace muon
