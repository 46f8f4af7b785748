// The GEMM kernel family: Y[M, N] = dequant(Xq) . dequant(Wq)^T for M <= 32.
//
// ai-radar.it, "Helion nel backend vLLM: un solo GEMM, tuning per forma e
// guadagni fino al 10%", paragraphs 2-3: Standard, Split-K and Swap-AB are
// tunable parameters of one GEMM implementation; split_k is a power of two up
// to 256.  Here they are template and launch parameters of one kernel:
//
//   grid   (ceil(N / (16*WN)), split_k); block 64*WN*WK threads.
//   wave   (wn, wk): weight rows n0 .. n0+15, n0 = tile*16*WN + 16*wn, and
//          the wk-th slice of the workgroup's K range.
//   K loop one MFMA per K-step (64 bytes of K for int8, 128 for E4M3FN); each
//          lane streams its weight row's bytes straight from HBM into MFMA
//          operand registers with 16-byte loads (no LDS for weights: every
//          weight byte is used by at most 32 tokens, so there is no reuse to
//          stage), double-buffered UNROLL K-steps deep.  Activation rows are
//          loaded the same way (they are tiny and stay in L2).
//   Swap-AB SWAP=0: A = activations, B = weights^T, C[m][n];
//          SWAP=1: A = weights, B = activations^T, C[n][m] = (Wq . Xq^T)^T.
//          The MFMA work is identical (square 16x16 tiles); what changes is
//          the accumulator-to-lane map and so the epilogue's store pattern.
//   WK     waves splitting K inside the workgroup are summed through LDS in
//          fixed wave order.
//   Split-K  each workgroup writes its partial tile to the workspace; the
//          last workgroup of a tile to arrive (arrival counter) sums the
//          partials in split order, runs the epilogue and resets the counter.
//          The fixed order makes results run-to-run deterministic; empty
//          splits (split_k > number of K-steps) contribute zeros.
//   Block_FP8  K-step = one 128-wide group: each group's MFMA starts from
//          zero and is added into the fp32 accumulator times
//          sx[m, g] * sw[n / 128, g].
//   Epilogue  y = bf16(acc * sx[m] * sw[n]) for the per-token formats,
//          bf16(acc) for Block_FP8, or the raw accumulator (test mode).
//
// Rows beyond M (padding of the 16-row MFMA tile) and beyond N (ragged last
// tile) read a clamped valid row; their outputs are never stored.  A ragged
// K tail (K % KSTEP != 0, K % 16 == 0) is one masked K-step.
#pragma once
#include <type_traits>

#include "w8_device.hpp"
#include "w8_launch.hpp"

namespace w8 {

template <int FMT>
struct Traits;
template <>
struct Traits<W8A8_INT8> {
  static constexpr int KSTEP = 64;
  typedef v4i Frag;
  typedef v4i Acc;
};
template <>
struct Traits<FP8_DYNAMIC> {
  static constexpr int KSTEP = 128;
  typedef v8i Frag;
  typedef v4f Acc;
};
template <>
struct Traits<BLOCK_FP8> {
  static constexpr int KSTEP = 128;
  typedef v8i Frag;
  typedef v4f Acc;
};

// The lane's bytes of K-step kk of one row: [kk*KSTEP + 16g, +16) and, for
// E4M3FN, also [kk*KSTEP + 64 + 16g, +16).  row points at row + 16*g.
template <int FMT>
__device__ __forceinline__ typename Traits<FMT>::Frag load_frag(const uint8_t* row, int kk) {
  if constexpr (FMT == W8A8_INT8) {
    return *reinterpret_cast<const v4i*>(row + (long long)kk * 64);
  } else {
    const v4i lo = *reinterpret_cast<const v4i*>(row + (long long)kk * 128);
    const v4i hi = *reinterpret_cast<const v4i*>(row + (long long)kk * 128 + 64);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// Same, for the ragged last K-step: 16-byte chunks at or beyond K read as 0.
template <int FMT>
__device__ __forceinline__ typename Traits<FMT>::Frag load_frag_tail(const uint8_t* row, int kk,
                                                                     int k_lane, int K) {
  const v4i z = {0, 0, 0, 0};
  if constexpr (FMT == W8A8_INT8) {
    const int c = kk * 64 + k_lane;
    return c < K ? *reinterpret_cast<const v4i*>(row + (long long)kk * 64) : z;
  } else {
    const int c = kk * 128 + k_lane;
    const v4i lo = c < K ? *reinterpret_cast<const v4i*>(row + (long long)kk * 128) : z;
    const v4i hi = c + 64 < K ? *reinterpret_cast<const v4i*>(row + (long long)kk * 128 + 64) : z;
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <int FMT, int SWAP>
__device__ __forceinline__ typename Traits<FMT>::Acc mma(typename Traits<FMT>::Frag w,
                                                        typename Traits<FMT>::Frag x,
                                                        typename Traits<FMT>::Acc c) {
  if constexpr (FMT == W8A8_INT8) {
    return SWAP ? mfma_i8(w, x, c) : mfma_i8(x, w, c);
  } else {
    return SWAP ? mfma_f8(w, x, c) : mfma_f8(x, w, c);
  }
}

template <int FMT, int MB, int WN, int WK, int U, int SWAP>
__global__ __launch_bounds__(64 * WN * WK) void gemm_kernel(GemmArgs a) {
  typedef typename Traits<FMT>::Frag Frag;
  typedef typename Traits<FMT>::Acc Acc;
  constexpr bool BLOCK = (FMT == BLOCK_FP8);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % WN, wk = wave / WN;
  const int r = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int n0 = tile * (16 * WN) + 16 * wn;

  // Row pointers (clamped rows for the M padding and the ragged N tile).
  const uint8_t* wrow = a.wq + (long long)min(n0 + r, a.N - 1) * a.ldw + 16 * g;
  const uint8_t* xrow[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) xrow[b] = a.xq + (long long)min(16 * b + r, a.M - 1) * a.ldq + 16 * g;

  // Block_FP8 scale pointers for this lane: sw row of the 128-row block, and
  // the sx rows of the accumulator elements the lane holds (SWAP: one m per
  // lane; standard: four).
  constexpr int SXN = SWAP ? 1 : 4;
  const float* swrow = nullptr;
  const float* sxrow[MB][SXN];
  if constexpr (BLOCK) {
    swrow = a.sw + (long long)(min(n0, a.N - 1) / kGroup) * a.sgroups;
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < SXN; ++i) {
        const int m = SWAP ? 16 * b + r : 16 * b + 4 * g + i;
        sxrow[b][i] = a.sx + (long long)min(m, a.M - 1) * a.sgroups;
      }
  }

  // Epilogue scales of the per-token formats, loaded now so their latency
  // hides under the K loop instead of adding a round trip at the end.
  float ep_sx[MB][SXN], ep_sw[4 / SXN];
  if constexpr (!BLOCK) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < SXN; ++i)
        ep_sx[b][i] = a.sx[min(SWAP ? 16 * b + r : 16 * b + 4 * g + i, a.M - 1)];
#pragma unroll
    for (int i = 0; i < 4 / SXN; ++i)
      ep_sw[i] = a.sw[min(SWAP ? n0 + 4 * g + i : n0 + r, a.N - 1)];
  }

  // K-steps of this split, then of this wave.
  // (32-bit: the host guarantees split_k * ksteps < 2^31.)
  const int ka = (int)((unsigned)(split * a.ksteps) / (unsigned)a.split_k);
  const int kb = (int)((unsigned)((split + 1) * a.ksteps) / (unsigned)a.split_k);
  const int la = ka + (kb - ka) * wk / WK;
  const int lb = ka + (kb - ka) * (wk + 1) / WK;
  const int lfull = min(lb, a.kfull);

  Acc acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = Acc{0, 0, 0, 0};

  // A stage is U consecutive K-steps.  The wave's full K-steps [la, lfull)
  // are covered by ns whole stages ending at lfull; the first stage may
  // start before la, and its steps below la load a clamped (valid) address
  // and are zeroed before their MFMA, so every load of a stage is issued at
  // once and no K-step is ever processed alone.
  struct Stage {
    Frag w[U];
    Frag x[U][MB];
    float sw[BLOCK ? U : 1];
    float sx[BLOCK ? U : 1][MB][SXN];
  };
  auto load_stage = [&](Stage& st, int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = max(k0 + u, la);
      st.w[u] = load_frag<FMT>(wrow, k);
#pragma unroll
      for (int b = 0; b < MB; ++b) st.x[u][b] = load_frag<FMT>(xrow[b], k);
      if constexpr (BLOCK) {
        st.sw[u] = swrow[k];
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int i = 0; i < SXN; ++i) st.sx[u][b][i] = sxrow[b][i][k];
      }
    }
  };
  // MASK: the first stage, whose steps below la are zeroed.
  auto run_stage = [&](const Stage& st, int k0, auto mask) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const Frag zero = {};
      const Frag w = (decltype(mask)::value && k0 + u < la) ? zero : st.w[u];
      if constexpr (BLOCK) {
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const Acc p = mma<FMT, SWAP>(w, st.x[u][b], Acc{0, 0, 0, 0});
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[b][i] += p[i] * (st.sx[u][b][SWAP ? 0 : i] * st.sw[u]);
        }
      } else {
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[b] = mma<FMT, SWAP>(w, st.x[u][b], acc[b]);
      }
    }
  };
  const std::true_type masked;
  const std::false_type whole;

  // Stages alternate between register sets A and B: the loads of stage s+1
  // are issued before stage s feeds the MFMAs.
  const int ns = (max(lfull - la, 0) + U - 1) / U;
  if (ns > 0) {
    const int k0 = lfull - ns * U;
    Stage A, B;
    load_stage(A, k0);
    if (ns == 1) {
      run_stage(A, k0, masked);
    } else {
      load_stage(B, k0 + U);
      run_stage(A, k0, masked);
      int s = 1;  // B holds stage s
      for (; s + 2 <= ns - 1; s += 2) {
        load_stage(A, k0 + (s + 1) * U);
        run_stage(B, k0 + s * U, whole);
        load_stage(B, k0 + (s + 2) * U);
        run_stage(A, k0 + (s + 1) * U, whole);
      }
      if (s + 1 <= ns - 1) {
        load_stage(A, k0 + (s + 1) * U);
        run_stage(B, k0 + s * U, whole);
        run_stage(A, k0 + (s + 1) * U, whole);
      } else {
        run_stage(B, k0 + s * U, whole);
      }
    }
  }
  // The ragged K tail (K % KSTEP != 0; never for Block_FP8, whose K is a
  // multiple of its 128-byte K-step) belongs to the wave that owns step kfull.
  if (!BLOCK && lb > a.kfull && la < lb) {
    Frag xs[MB];
    const Frag ws = load_frag_tail<FMT>(wrow, a.kfull, 16 * g, a.K);
#pragma unroll
    for (int b = 0; b < MB; ++b) xs[b] = load_frag_tail<FMT>(xrow[b], a.kfull, 16 * g, a.K);
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = mma<FMT, SWAP>(ws, xs[b], acc[b]);
  }

  // Sum the WK waves of each wn through LDS, in wave order.
  if constexpr (WK > 1) {
    __shared__ Acc red[(WK - 1) * WN * MB * 64];
    if (wk > 0) {
#pragma unroll
      for (int b = 0; b < MB; ++b) red[(((wk - 1) * WN + wn) * MB + b) * 64 + lane] = acc[b];
    }
    __syncthreads();
    if (wk == 0) {
      for (int j = 1; j < WK; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[b] += red[(((j - 1) * WN + wn) * MB + b) * 64 + lane];
    }
  }

  // Split-K: publish the partial; the last workgroup of the tile reduces.
  // Protocol (no L2 writeback or invalidate): the partials are written with
  // agent-scope atomic stores, which write through this XCD's L2 to the
  // device-coherent level; s_waitcnt waits until every one of them is
  // acknowledged before the workgroup counts itself in; the last workgroup
  // to arrive reads the partials with agent-scope atomic loads, which are
  // served from the device-coherent level, so it sees every split's data.
  // Partial layout: fragment f = ((tile*S + split)*WN + wn)*MB + b holds
  // 4 x 64 words, word (f*4 + i)*64 + lane, so each of the four stores of a
  // wave writes 256 contiguous bytes.
  if (a.split_k > 1) {
    typedef decltype(acc[0][0]) Elem;
    typedef typename std::remove_cv<typename std::remove_reference<Elem>::type>::type Word;
    Word* part = reinterpret_cast<Word*>(a.part);
    const long long frag0 = (long long)tile * a.split_k;
    if (wk == 0) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(part + ((((frag0 + split) * WN + wn) * MB + b) * 4 + i) * 64 + lane,
                             acc[b][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int is_last;
    if (threadIdx.x == 0) {
      const unsigned prev = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      is_last = (prev == (unsigned)(a.split_k - 1));
    }
    __syncthreads();
    if (!is_last) return;
    if (wk == 0) {
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[b] = Acc{0, 0, 0, 0};
      for (int s = 0; s < a.split_k; ++s)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[b][i] += __hip_atomic_load(
                part + ((((frag0 + s) * WN + wn) * MB + b) * 4 + i) * 64 + lane, __ATOMIC_RELAXED,
                __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (wk != 0) return;

  // Epilogue.
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = SWAP ? 16 * b + r : 16 * b + 4 * g + i;
      const int n = SWAP ? n0 + 4 * g + i : n0 + r;
      if (m < a.M && n < a.N) {
        const long long o = (long long)m * a.ldo + n;
        if (a.out_mode) {
          if constexpr (FMT == W8A8_INT8)
            reinterpret_cast<int*>(a.out)[o] = acc[b][i];
          else
            reinterpret_cast<float*>(a.out)[o] = acc[b][i];
        } else {
          float y;
          if constexpr (BLOCK) {
            y = acc[b][i];
          } else {
            const float sxm = ep_sx[b][SWAP ? 0 : i], swn = ep_sw[SWAP ? i : 0];
            if constexpr (FMT == W8A8_INT8)
              y = (float)acc[b][i] * sxm * swn;
            else
              y = acc[b][i] * sxm * swn;
          }
          reinterpret_cast<uint16_t*>(a.out)[o] = bf16_rne(y);
        }
      }
    }
}

template <int FMT, int MB, int WN, int WK, int U, int SWAP>
hipError_t launch_gemm(const GemmArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<FMT, MB, WN, WK, U, SWAP>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace w8
