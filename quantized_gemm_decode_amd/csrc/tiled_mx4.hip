// Tiled GEMM instantiations for MXFP4 weights (E2M1, 1 KB packed tiles) with
// MXFP8 activations: packed operands, register ring; the E8M0 block scales
// of both operands go to the scaled matrix-core instruction.
#include "tiled_gemm.hpp"

namespace qlk {
hipError_t tiled_dispatch_mx4(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                              bool probe_only) {
  return tiled_dispatch<FMT_MX4>(k, grid, lds, s, a, probe_only);
}
}  // namespace qlk
