// Tile-128 instantiation of the Newton-Schulz GEMM kernels (muon_gemm.h).
// Built with MFMA accumulators in ordinary vector registers: at this tile
// size they fit beside everything else, and the accumulator-register form
// made the compiler copy accumulators inside the K loop.
#include "muon_gemm.h"

namespace muon {

int launch_gram_128(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                   void* stream) {
  return launch_gram_t<128>(d, prefix, n, units, parity, stream);
}

int launch_gram2_128(const MatDesc* d, const int64_t* prefix, int n, int64_t units, float a,
                    float b, float c, void* stream) {
  return launch_gram2_t<128>(d, prefix, n, units, a, b, c, stream);
}

int launch_xupdate_128(const MatDesc* d, const int64_t* prefix, int n, int64_t units, int parity,
                      void* stream) {
  return launch_xupdate_t<128>(d, prefix, n, units, parity, stream);
}

}  // namespace muon
