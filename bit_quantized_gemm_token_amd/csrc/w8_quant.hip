// Activation and weight quantization kernels.
//
// ai-radar.it, "Helion nel backend vLLM: un solo GEMM, tuning per forma e
// guadagni fino al 10%", paragraph 1 (the formats) and paragraph 8
// (quantization as an auxiliary kernel beside the GEMM).  Every group uses
// s = amax / Qmax (an all-zero group takes s = 1) and codes
// round-to-nearest-even(x / s) with saturation.  s is the correctly rounded
// fp32 division (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt and without fast-math); x / s
// takes the reciprocal-and-correction form of encode8, which gives the
// codes of the correctly rounded quotient.
#include "w8_device.hpp"
#include "w8_launch.hpp"

namespace w8 {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kRowCache = 4;  // 16-byte chunks per thread kept in registers (K <= 8192)

// Per-token quantization: one workgroup per row.
template <bool INT8>
__global__ __launch_bounds__(kQuantThreads) void quant_token_kernel(QuantActArgs a) {
  const int m = blockIdx.x;
  const uint16_t* xr = a.x + (long long)m * a.ldx;
  uint8_t* qr = a.xq + (long long)m * a.ldq;
  const int nch = a.K / 8;
  const int t = threadIdx.x;

  v4u cache[kRowCache];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kRowCache; ++i) {
    const int c = t + i * kQuantThreads;
    cache[i] = v4u{0u, 0u, 0u, 0u};
    if (c < nch) cache[i] = *reinterpret_cast<const v4u*>(xr + 8 * c);
    amax = fmaxf(amax, absmax8(cache[i]));
  }
  for (int c = t + kRowCache * kQuantThreads; c < nch; c += kQuantThreads)
    amax = fmaxf(amax, absmax8(*reinterpret_cast<const v4u*>(xr + 8 * c)));

  __shared__ float red[kQuantThreads / 64];
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, red[w]);

  const float s = act_scale<INT8>(amax);
  const float rs = act_recip(s);
  if (t == 0) a.sx[m] = s;

#pragma unroll
  for (int i = 0; i < kRowCache; ++i) {
    const int c = t + i * kQuantThreads;
    if (c < nch) *reinterpret_cast<v2u*>(qr + 8 * c) = encode8<INT8>(cache[i], s, rs);
  }
  for (int c = t + kRowCache * kQuantThreads; c < nch; c += kQuantThreads)
    *reinterpret_cast<v2u*>(qr + 8 * c) =
        encode8<INT8>(*reinterpret_cast<const v4u*>(xr + 8 * c), s, rs);
}

// Per-group (1 x 128) E4M3FN quantization: 16 lanes per group, each lane one
// 16-byte chunk of 8 values; 16 groups per workgroup.
__global__ __launch_bounds__(kQuantThreads) void quant_group_kernel(QuantActArgs a) {
  const int G = a.K / kGroup;
  const int gid = blockIdx.x * (kQuantThreads / 16) + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool active = gid < a.M * G;
  const int m = active ? gid / G : 0;
  const int g = active ? gid % G : 0;
  const long long xo = (long long)m * a.ldx + g * kGroup + 8 * j;

  v4u v = v4u{0u, 0u, 0u, 0u};
  if (active) v = *reinterpret_cast<const v4u*>(a.x + xo);
  const float amax = seg16_max(absmax8(v));
  const float s = act_scale<false>(amax);
  if (active) {
    if (j == 0) a.sx[(long long)m * G + g] = s;
    *reinterpret_cast<v2u*>(a.xq + (long long)m * a.ldq + g * kGroup + 8 * j) =
        encode8<false>(v, s, act_recip(s));
  }
}

__device__ __forceinline__ float block_max(float v) {
  __shared__ float red[kQuantThreads / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; ++w) v = fmaxf(v, red[w]);
  return v;
}

__device__ __forceinline__ uint8_t e4m3_byte(float v) { return (uint8_t)(e4m3_pack4(v, 0.f, 0.f, 0.f) & 0xFFu); }

// Offline weight quantization, one E4M3FN scale per row (FP8_Dynamic).
__global__ __launch_bounds__(kQuantThreads) void quant_weight_row_kernel(QuantWeightArgs a) {
  const int n = blockIdx.x;
  const float* wr = a.w + (long long)n * a.ldw;
  float amax = 0.0f;
  for (int k = threadIdx.x; k < a.K; k += kQuantThreads) amax = fmaxf(amax, fabsf(wr[k]));
  amax = block_max(amax);
  const float s = (amax == 0.0f) ? 1.0f : amax / kQmaxE4M3;
  if (threadIdx.x == 0) a.sw[n] = s;
  uint8_t* qr = a.wq + (long long)n * a.ldq;
  for (int k = threadIdx.x; k < a.K; k += kQuantThreads) qr[k] = e4m3_byte(wr[k] / s);
}

// Offline weight quantization, one E4M3FN scale per 128 x 128 block (Block_FP8).
__global__ __launch_bounds__(kQuantThreads) void quant_weight_block_kernel(QuantWeightArgs a) {
  const int bn = blockIdx.y, bk = blockIdx.x;
  const int KB = gridDim.x;
  const int n0 = bn * kGroup, k0 = bk * kGroup;
  const int nr = min(kGroup, a.N - n0), kc = min(kGroup, a.K - k0);
  float amax = 0.0f;
  for (int e = threadIdx.x; e < nr * kc; e += kQuantThreads)
    amax = fmaxf(amax, fabsf(a.w[(long long)(n0 + e / kc) * a.ldw + k0 + e % kc]));
  amax = block_max(amax);
  const float s = (amax == 0.0f) ? 1.0f : amax / kQmaxE4M3;
  if (threadIdx.x == 0) a.sw[(long long)bn * KB + bk] = s;
  for (int e = threadIdx.x; e < nr * kc; e += kQuantThreads) {
    const long long row = n0 + e / kc;
    a.wq[row * a.ldq + k0 + e % kc] = e4m3_byte(a.w[row * a.ldw + k0 + e % kc] / s);
  }
}

}  // namespace

hipError_t launch_quantize_act(int fmt, const QuantActArgs& a, hipStream_t s) {
  if (fmt == BLOCK_FP8) {
    const int groups = a.M * (a.K / kGroup);
    const int blocks = (groups + kQuantThreads / 16 - 1) / (kQuantThreads / 16);
    hipLaunchKernelGGL(quant_group_kernel, dim3(blocks), dim3(kQuantThreads), 0, s, a);
  } else if (fmt == W8A8_INT8) {
    hipLaunchKernelGGL(quant_token_kernel<true>, dim3(a.M), dim3(kQuantThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(quant_token_kernel<false>, dim3(a.M), dim3(kQuantThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_weight(int fmt, const QuantWeightArgs& a, hipStream_t s) {
  if (fmt == BLOCK_FP8) {
    const int NB = (a.N + kGroup - 1) / kGroup, KB = (a.K + kGroup - 1) / kGroup;
    hipLaunchKernelGGL(quant_weight_block_kernel, dim3(KB, NB), dim3(kQuantThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(quant_weight_row_kernel, dim3(a.N), dim3(kQuantThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace w8
