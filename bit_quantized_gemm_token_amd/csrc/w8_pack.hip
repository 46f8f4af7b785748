// Offline packing of weight codes into the GEMM's MFMA-native layout (the
// "memory layout" choice of ai-radar.it, "Helion nel backend vLLM",
// paragraph 3).
#include "w8_gemm.hpp"

namespace w8 {

template <int KSTEP>
static void launch_pack(const uint8_t* w, long long ldw, int N, int K, uint8_t* out, int layout,
                        int spans, long long chunks, hipStream_t s) {
  const dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
  switch (layout) {
    case 1: hipLaunchKernelGGL((pack_weight_kernel<KSTEP, 1>), grid, block, 0, s, w, ldw, N, K, spans, out, chunks); break;
    case 2: hipLaunchKernelGGL((pack_weight_kernel<KSTEP, 2>), grid, block, 0, s, w, ldw, N, K, spans, out, chunks); break;
    case 4: hipLaunchKernelGGL((pack_weight_kernel<KSTEP, 4>), grid, block, 0, s, w, ldw, N, K, spans, out, chunks); break;
    default: hipLaunchKernelGGL((pack_weight_kernel<KSTEP, 8>), grid, block, 0, s, w, ldw, N, K, spans, out, chunks); break;
  }
}

hipError_t launch_pack_weight(int fmt, const uint8_t* w, long long ldw, int N, int K,
                              uint8_t* out, int layout, hipStream_t s) {
  const long long chunks = (long long)(packed_weight_bytes(fmt, N, K, layout) / 16);
  const int spans = layout_spans(fmt, K, layout);
  if (fmt == W8A8_INT8)
    launch_pack<64>(w, ldw, N, K, out, layout, spans, chunks, s);
  else
    launch_pack<128>(w, ldw, N, K, out, layout, spans, chunks, s);
  return hipGetLastError();
}

}  // namespace w8
