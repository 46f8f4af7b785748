// The read floor: one launch that streams `bytes` of device memory and does
// nothing else.  The GEMM moves its weights the same way (16-byte loads,
// each byte read once, non-temporal), so the time of this kernel for the
// same bytes, graph-replayed over the same rotating buffers, is the bound a
// one-launch GEMM can approach; the benchmark reports each GEMM's time
// against it.
//
// Access pattern: 1 KiB chunks (one load instruction of a wave, lane l
// reading 16 bytes at +16 l), dealt to the waves of the grid interleaved --
// wave w reads chunks w, w + W, w + 2W, ... (W waves in all) -- so the waves
// of one moment read neighbouring memory; DEPTH chunks per wave in flight.
// Each wave XORs what it read and writes one word of `sink`, so no load is
// dead code and, like a GEMM, the launch ends with a store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w8_internal.hpp"

namespace w8 {
namespace {

typedef unsigned int u4 __attribute__((ext_vector_type(4)));

template <int DEPTH>
__global__ void read_floor_kernel(const u4* __restrict__ src, long long nchunks,
                                  unsigned* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long long W = (long long)gridDim.x * (blockDim.x >> 6);
  const long long w = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const u4* p = src + lane;
  u4 acc = {0u, 0u, 0u, 0u};
  for (long long c = w; c < nchunks; c += DEPTH * W) {
    u4 v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      v[d] = c + d * W < nchunks ? __builtin_nontemporal_load(p + (c + d * W) * 64)
                                 : u4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= v[d];
  }
  // the wave's XOR: within each row of 16 lanes by DPP moves, then across
  // the four rows by lane reads (no LDS round trips)
  int x = (int)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  x ^= __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x ^= __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x ^= __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x ^= __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
  x = __builtin_amdgcn_readlane(x, 0) ^ __builtin_amdgcn_readlane(x, 16) ^
      __builtin_amdgcn_readlane(x, 32) ^ __builtin_amdgcn_readlane(x, 48);
  if (lane == 0) sink[w] = (unsigned)x;
}

}  // namespace
}  // namespace w8

using namespace w8;

extern "C" w8_status w8_read_floor(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                                   int grid, int waves, int depth, w8_stream stream) {
  if (!src || !sink) return fail(W8_E_INVALID, "null device pointer");
  if (((uintptr_t)src % 16) || ((uintptr_t)sink % 4))
    return fail(W8_E_INVALID, "src must be 16-byte and sink 4-byte aligned");
  if (bytes < 1024 || bytes % 1024)
    return fail(W8_E_INVALID, "bytes must be a positive multiple of 1024");
  if (grid < 1 || grid > 65535) return fail(W8_E_INVALID, "grid must be in [1, 65535]");
  if (waves != 1 && waves != 2 && waves != 4 && waves != 8 && waves != 16)
    return fail(W8_E_INVALID, "waves must be 1, 2, 4, 8 or 16");
  if ((size_t)grid * (size_t)waves * 4 > sink_bytes)
    return fail(W8_E_INVALID, "sink must hold grid * waves 4-byte words");
  w8_status st = check_device();
  if (st) return st;
  const long long nchunks = (long long)(bytes / 1024);
  const u4* s4 = static_cast<const u4*>(src);
  unsigned* out = static_cast<unsigned*>(sink);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(grid), b(64 * waves);
  switch (depth) {
    case 1: hipLaunchKernelGGL(read_floor_kernel<1>, g, b, 0, s, s4, nchunks, out); break;
    case 2: hipLaunchKernelGGL(read_floor_kernel<2>, g, b, 0, s, s4, nchunks, out); break;
    case 4: hipLaunchKernelGGL(read_floor_kernel<4>, g, b, 0, s, s4, nchunks, out); break;
    case 8: hipLaunchKernelGGL(read_floor_kernel<8>, g, b, 0, s, s4, nchunks, out); break;
    default: return fail(W8_E_INVALID, "depth must be 1, 2, 4 or 8");
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("read floor launch", e));
  return ok();
}
