// Decode GEMM instantiations for MXFP4 weights with MXFP8 activations (packed
// operands; the E8M0 block scales go to the scaled matrix-core instruction).
#include "decode_gemm.hpp"

namespace qlk {
hipError_t decode_dispatch_mx4(const DecodeKey& k, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                              const DecodeArgs& a, bool probe_only) {
  return decode_dispatch<FMT_MX4>(k, grid, block, lds, s, a, probe_only);
}
}  // namespace qlk
