// Decode GEMM instantiations for one format (split per format so the
// instantiation tables compile in parallel).
#include "decode_gemm.hpp"

namespace qlk {
hipError_t decode_dispatch_fp8(const DecodeKey& k, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                              const DecodeArgs& a, bool probe_only) {
  return decode_dispatch<FMT_FP8>(k, grid, block, lds, s, a, probe_only);
}
}  // namespace qlk
