// Tiled GEMM instantiations for one format (one translation unit per format
// so the instantiation tables compile in parallel).
#include "tiled_gemm.hpp"

namespace qlk {
hipError_t tiled_dispatch_int8(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                               bool probe_only) {
  return tiled_dispatch<FMT_INT8>(k, grid, lds, s, a, probe_only);
}
}  // namespace qlk
