// A plain streaming read of device memory: the time a buffer of a GEMM's
// operand size takes to cross from HBM with nothing else to do, on this
// device.  A weight-streaming GEMM is measured against it (the HBM peak is
// not reachable by any kernel at the sizes of decode GEMMs, where launch and
// ramp take a fixed share).  Each workgroup reads a contiguous slice in
// 16-byte nontemporal loads, 4 or 8 in flight per lane.  In its checking
// mode each workgroup writes the wrapping 32-bit sum of the words it read, so
// a test can check that every byte was read exactly once; the timing mode
// writes nothing in practice.
#include "decode_args.hpp"
#include "device_common.hpp"

namespace qlk {

constexpr int kStreamThreads = 256;

// Workgroup w reads the contiguous slice [w*per, min(n16, (w+1)*per)) of
// 16-byte pieces, UNROLL pieces in flight per lane (a workgroup load covers
// 4 KB, so UNROLL consecutive 4 KB spans are in flight per workgroup).
// CHECK: every workgroup reduces its lanes' sums and writes one word.
// Otherwise a lane writes its own sum only if it equals a fixed constant:
// the loads stay live, and the kernel's end waits for no writes (a plain
// read, as the ceiling should be).
constexpr uint32_t kStreamMagic = 0x9E3779B9u;

template <int UNROLL, bool CHECK>
__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                                      uint32_t* __restrict__ sink) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t b = (uint64_t)blockIdx.x * per;
  const uint64_t e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  for (uint64_t i = b + threadIdx.x; i < e; i += (uint64_t)kStreamThreads * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint64_t j = i + (uint64_t)u * kStreamThreads;
      v[u] = j < e ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  if constexpr (CHECK) {
    __shared__ uint32_t part[kStreamThreads / 64];
    for (int o = 32; o > 0; o >>= 1) acc += (uint32_t)__shfl_xor((int)acc, o, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t s = 0;
      for (int w = 0; w < kStreamThreads / 64; ++w) s += part[w];
      sink[blockIdx.x] = s;
    }
  } else {
    if (acc == kStreamMagic) sink[blockIdx.x] = acc;
  }
}

hipError_t launch_stream_read(const void* src, uint64_t bytes, int workgroups, int unroll, bool check,
                              uint32_t* sink, hipStream_t s) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const dim3 grid((unsigned)workgroups), block(kStreamThreads);
  const uint64_t n16 = bytes / 16u;
  if (unroll == 4 && check)
    hipLaunchKernelGGL((stream_read_kernel<4, true>), grid, block, 0, s, p, n16, sink);
  else if (unroll == 4)
    hipLaunchKernelGGL((stream_read_kernel<4, false>), grid, block, 0, s, p, n16, sink);
  else if (check)
    hipLaunchKernelGGL((stream_read_kernel<8, true>), grid, block, 0, s, p, n16, sink);
  else
    hipLaunchKernelGGL((stream_read_kernel<8, false>), grid, block, 0, s, p, n16, sink);
  return hipGetLastError();
}

// Broadcast read: workgroup w reads the w-th contiguous slice of `p` (as
// above) and, interleaved with it piece for piece, the whole block `b` --
// the bytes each compute unit of a weight-streaming GEMM without a K split
// must load: its share of the weights (nontemporal, from HBM) and every
// token's activations (ordinary loads; every workgroup reads the same block,
// so after the first it comes from L2).  Launched with one workgroup per
// compute unit, its time is the ceiling of that decomposition on this
// device.  NT threads, UNROLL pieces of each stream in flight per lane.
template <int UNROLL, int NT, bool CHECK>
__global__ void __launch_bounds__(NT) stream_bcast_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                           const u32x4* __restrict__ b, uint32_t b16,
                                                           uint32_t* __restrict__ sink) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t beg = (uint64_t)blockIdx.x * per;
  const uint64_t e = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  uint64_t i = beg + threadIdx.x;
  uint32_t j = threadIdx.x;
  while (i < e || j < b16) {
    u32x4 v[UNROLL], a[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint64_t x = i + (uint64_t)u * NT;
      v[u] = x < e ? __builtin_nontemporal_load(p + x) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t y = j + (uint32_t)(u * NT);
      a[u] = y < b16 ? b[y] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w + a[u].x + a[u].y + a[u].z + a[u].w;
    i += (uint64_t)NT * UNROLL;
    j += (uint32_t)(NT * UNROLL);
  }
  if constexpr (CHECK) {
    __shared__ uint32_t part[NT / 64];
    for (int o = 32; o > 0; o >>= 1) acc += (uint32_t)__shfl_xor((int)acc, o, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t s = 0;
      for (int w = 0; w < NT / 64; ++w) s += part[w];
      sink[blockIdx.x] = s;
    }
  } else {
    if (acc == kStreamMagic) sink[blockIdx.x] = acc;
  }
}

template <int UNROLL, int NT>
static hipError_t launch_bcast(const u32x4* p, uint64_t n16, const u32x4* b, uint32_t b16, int workgroups,
                               bool check, uint32_t* sink, hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(NT);
  if (check)
    hipLaunchKernelGGL((stream_bcast_kernel<UNROLL, NT, true>), grid, block, 0, s, p, n16, b, b16, sink);
  else
    hipLaunchKernelGGL((stream_bcast_kernel<UNROLL, NT, false>), grid, block, 0, s, p, n16, b, b16, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read_bcast(const void* src, uint64_t bytes, const void* bcast, uint64_t bcast_bytes,
                                    int workgroups, int threads, int unroll, bool check, uint32_t* sink,
                                    hipStream_t s) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const u32x4* b = reinterpret_cast<const u32x4*>(bcast);
  const uint64_t n16 = bytes / 16u;
  const uint32_t b16 = (uint32_t)(bcast_bytes / 16u);
  if (unroll == 2) {
    if (threads == 256) return launch_bcast<2, 256>(p, n16, b, b16, workgroups, check, sink, s);
    if (threads == 512) return launch_bcast<2, 512>(p, n16, b, b16, workgroups, check, sink, s);
    return launch_bcast<2, 1024>(p, n16, b, b16, workgroups, check, sink, s);
  }
  if (threads == 256) return launch_bcast<4, 256>(p, n16, b, b16, workgroups, check, sink, s);
  if (threads == 512) return launch_bcast<4, 512>(p, n16, b, b16, workgroups, check, sink, s);
  return launch_bcast<4, 1024>(p, n16, b, b16, workgroups, check, sink, s);
}

}  // namespace qlk
