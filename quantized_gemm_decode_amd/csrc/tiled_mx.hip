// Tiled GEMM instantiations for MXFP8 (packed operands, register ring; the
// E8M0 block scales go to the scaled matrix-core instruction).
#include "tiled_gemm.hpp"

namespace qlk {
hipError_t tiled_dispatch_mx(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                             bool probe_only) {
  return tiled_dispatch<FMT_MX>(k, grid, lds, s, a, probe_only);
}
}  // namespace qlk
