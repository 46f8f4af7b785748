// Offline packing of weight codes into the GEMM's MFMA-native layout (the
// "memory layout" choice of ai-radar.it, "Helion nel backend vLLM",
// paragraph 3).
#include "w8_gemm.hpp"

namespace w8 {

hipError_t launch_pack_weight(int fmt, const uint8_t* w, long long ldw, int N, int K,
                              uint8_t* out, hipStream_t s) {
  const long long chunks = (long long)(packed_weight_bytes(fmt, N, K) / 16);
  const int blocks = (int)((chunks + 255) / 256);
  if (fmt == W8A8_INT8)
    hipLaunchKernelGGL(pack_weight_kernel<64>, dim3(blocks), dim3(256), 0, s, w, ldw, N, K,
                       (K + 63) / 64, out, chunks);
  else
    hipLaunchKernelGGL(pack_weight_kernel<128>, dim3(blocks), dim3(256), 0, s, w, ldw, N, K,
                       (K + 127) / 128, out, chunks);
  return hipGetLastError();
}

}  // namespace w8
