// Device-side helpers for gfx950: vector types, 8-bit encoders, bf16
// rounding, wavefront reductions and the two MFMA forms the GEMM uses.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

enum Fmt { FP8_DYNAMIC = 0, W8A8_INT8 = 1, BLOCK_FP8 = 2 };

constexpr float kQmaxE4M3 = 448.0f;  // largest finite OCP E4M3FN magnitude
constexpr float kQmaxInt8 = 127.0f;  // symmetric int8 range [-127, 127]
constexpr int kGroup = 128;          // Block_FP8 group / block edge

// ---------------------------------------------------------------- codecs --
// Saturating E4M3FN encode of four floats, packed little-endian into a dword.
// v_cvt_pk_fp8_f32 rounds to nearest even in the OCP E4M3FN format on gfx950;
// the explicit clamp to +-448 gives saturation (the sign of zero is kept by
// v_max/v_min, so -0 and negative underflow encode as 0x80).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kQmaxE4M3), kQmaxE4M3);
  b = fminf(fmaxf(b, -kQmaxE4M3), kQmaxE4M3);
  c = fminf(fmaxf(c, -kQmaxE4M3), kQmaxE4M3);
  d = fminf(fmaxf(d, -kQmaxE4M3), kQmaxE4M3);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// int8 encode: round to nearest even, clamp to [-127, 127].
__device__ __forceinline__ uint32_t i8_byte(float v) {
  float r = fminf(fmaxf(__builtin_rintf(v), -kQmaxInt8), kQmaxInt8);
  return (uint32_t)((int)r) & 0xFFu;
}

__device__ __forceinline__ uint32_t i8_pack4(float a, float b, float c, float d) {
  return i8_byte(a) | (i8_byte(b) << 8) | (i8_byte(c) << 16) | (i8_byte(d) << 24);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------ activation codes --
// The activation quantizer's per-element steps, shared by the standalone
// quantize kernels and the GEMM's fused-quantization staging so both give
// the same codes: amax of eight bf16 values (one 16-byte chunk), and eight
// bf16 values -> eight codes with code = encode(x / s).
__device__ __forceinline__ float absmax8(v4u v) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_lo(v[i])));
    m = fmaxf(m, fabsf(bf16_hi(v[i])));
  }
  return m;
}

// Scale of a group with absolute maximum amax (an all-zero group takes 1).
template <bool INT8>
__device__ __forceinline__ float act_scale(float amax) {
  return (amax == 0.0f) ? 1.0f : amax / (INT8 ? kQmaxInt8 : kQmaxE4M3);
}

// The quotient x / s is taken without a per-element division: with r the
// correctly rounded reciprocal of s, q0 = x*r, the residual x - q0*s is
// exact in one FMA, and q0 + residual*r is the correctly rounded quotient
// whenever nothing underflows (Markstein's correction step).  Where x is
// subnormal the two may differ in the last place, but for every scale
// s >= 2^-100 and every bf16 x with |x| <= the amax behind s they give the
// same E4M3FN and int8 code (checked exhaustively on the host).  Smaller
// scales (act_recip returns 0) divide.  The sign is copied from x so a
// negative zero keeps its code.  (The library is built without fast-math
// and with -fhip-fp32-correctly-rounded-divide-sqrt, so 1/s and x/s are
// correctly rounded.)
__device__ __forceinline__ float act_recip(float s) { return s >= 0x1p-100f ? 1.0f / s : 0.0f; }

__device__ __forceinline__ float act_quot(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
}

// Eight bf16 values -> eight codes; r = act_recip(s).
template <bool INT8>
__device__ __forceinline__ v2u encode8(v4u v, float s, float r) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
  if (r != 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = act_quot(f[i], s, r);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] / s;
  }
  v2u o;
  if (INT8) {
    o[0] = i8_pack4(f[0], f[1], f[2], f[3]);
    o[1] = i8_pack4(f[4], f[5], f[6], f[7]);
  } else {
    o[0] = e4m3_pack4(f[0], f[1], f[2], f[3]);
    o[1] = e4m3_pack4(f[4], f[5], f[6], f[7]);
  }
  return o;
}

// ------------------------------------------------------------- reductions --
// Lane moves within a row of 16 lanes by DPP (a VALU operand modifier: no
// LDS round trip, unlike a lane shuffle).  gfx9 DPP controls: quad_perm
// [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141
// (lane i <-> 7 - i within each 8), row_mirror = 0x140 (i <-> 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Max over aligned segments of 16 lanes (every lane gets its segment's max):
// pairs, then quads, then halves, then the row.
__device__ __forceinline__ float seg16_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));
  v = fmaxf(v, dpp_move<0x4E>(v));
  v = fmaxf(v, dpp_move<0x141>(v));
  v = fmaxf(v, dpp_move<0x140>(v));
  return v;
}

// Max over the 64 lanes of a wavefront (every lane gets the result): the
// four rows' maxima, read from one lane of each row.
__device__ __forceinline__ float wave_max(float v) {
  v = seg16_max(v);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ------------------------------------------------- device-coherent I/O --
// Buffer loads and stores of 16 bytes a lane with the agent-scope cache
// policy (SC1): the same bits the compiler sets on agent-scope atomic loads
// and stores, so a store is written through to the level the whole device
// shares and a load is served from it, whichever XCD the other side ran on.
// One instruction moves 1 KiB of a wave where the 4-byte atomic forms would
// take four.  `base` must be 4-byte aligned and the offsets below `bytes`.
constexpr int kCpolAgent = 16;  // SC1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ v4i coherent_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolAgent);
}
__device__ __forceinline__ void coherent_store16(__amdgpu_buffer_rsrc_t r, int off, v4i v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolAgent);
}

// ------------------------------------------------------------------- MFMA --
// 16x16 output tile; lane l holds column l%16, rows 4*(l/16) .. 4*(l/16)+3.
// A and B operands: lane l supplies row (A) / column (B) l%16 and one slice
// of K selected by l/16; both operands use the same lane->K assignment, so
// loading the same K bytes of an activation row and a weight row into the
// same lane slot pairs them correctly whatever the in-register K order is.

// int8 x int8 -> int32, K = 64 (16 bytes per lane per operand).
__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// E4M3FN x E4M3FN -> fp32, K = 128 (32 bytes per lane per operand).  Format
// selectors 0/0 pick FP8 E4M3 for both operands; zero scale operands select
// the unscaled v_mfma_f32_16x16x128_f8f6f4.
__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace w8
