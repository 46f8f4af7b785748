// The GEMM kernel family: Y[M, N] = dequant(Xq) . dequant(Wq)^T for M <= 32.
//
// ai-radar.it, "Helion nel backend vLLM: un solo GEMM, tuning per forma e
// guadagni fino al 10%", paragraphs 2-3: Standard, Split-K and Swap-AB are
// tunable parameters of one GEMM implementation; split_k is a power of two up
// to 256; the search also covers memory layout.  Here they are template and
// launch parameters of one kernel:
//
//   grid   ceil(N / (16*NB)) * split_k workgroups of 64*WK threads; the
//          split index varies fastest.  Workgroups are dealt round-robin to
//          the 8 XCDs, each with its own L2, so with split_k a power of two
//          an XCD sees only split_k/8 K ranges (split_k >= 8) or one (split_k
//          < 8), and fetches only those activation columns instead of all K.
//   wave   wk owns the workgroup's NB blocks of 16 weight rows
//          (n0 = tile*16*NB) over the wk-th slice of the workgroup's K range.
//   K loop one MFMA per K-step and row block (64 bytes of K for int8, 128 for
//          E4M3FN); each lane streams its weight bytes straight from HBM into
//          MFMA operand registers with 16-byte loads (no LDS for weights:
//          every weight byte meets at most 32 tokens, so there is nothing to
//          reuse), U K-steps per stage, two stages in flight.  The activation
//          fragment of a K-step is loaded once and reused by the NB row
//          blocks (activations are tiny and stay in L2).
//   layout PACKED=0: Wq row-major [N, K] (row stride ldw); a load instruction
//          reads 64 contiguous bytes of 16 rows.  PACKED=1: the MFMA-native
//          layout written by the weight packer: the 16 x KSTEP bytes of one
//          (row block, K-step) fragment are stored in lane order, so every
//          load instruction reads 1 KiB contiguous and a wave's whole K range
//          is one contiguous run; rows and K are zero-padded to whole
//          fragments.  Packed loads are non-temporal (each line is read once).
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

// Row-major operand: the lane's bytes of K-step kk of one row are
// [kk*KSTEP + 16g, +16) and, for E4M3FN, also [kk*KSTEP + 64 + 16g, +16).
// `row` points at row + 16*g.
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

// Packed operand: fragment (row block, K-step kk) of 16 x KSTEP bytes; the
// lane's 16 bytes of load instruction j are at j*1024 + 16*lane.  `frag`
// points at the row block's first fragment + 16*lane.
template <int FMT>
__device__ __forceinline__ typename Traits<FMT>::Frag load_packed(const uint8_t* frag, int kk) {
  constexpr int KSTEP = Traits<FMT>::KSTEP;
  const uint8_t* p = frag + (long long)kk * (16 * KSTEP);
  if constexpr (FMT == W8A8_INT8) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
  } else {
    const v4i lo = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
    const v4i hi = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p + 1024));
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

template <int FMT, int MB, int NB, int WK, int U, int SWAP, int PACKED>
__global__ __launch_bounds__(64 * WK) void gemm_kernel(GemmArgs a) {
  typedef typename Traits<FMT>::Frag Frag;
  typedef typename Traits<FMT>::Acc Acc;
  constexpr int KSTEP = Traits<FMT>::KSTEP;
  constexpr bool BLOCK = (FMT == BLOCK_FP8);

  const int lane = threadIdx.x & 63;
  const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int split = (int)(blockIdx.x & (unsigned)(a.split_k - 1));
  const int tile = (int)(blockIdx.x >> a.split_shift);
  const int n0 = tile * 16 * NB;

  // Weight pointers of the NB row blocks (clamped for the ragged N tile).
  const uint8_t* wptr[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if constexpr (PACKED) {
      const int nb = min(tile * NB + j, (a.N + 15) / 16 - 1);
      wptr[j] = a.wq + (long long)nb * a.ksteps * (16 * KSTEP) + 16 * lane;
    } else {
      wptr[j] = a.wq + (long long)min(n0 + 16 * j + r, a.N - 1) * a.ldw + 16 * g;
    }
  }
  const uint8_t* xrow[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) xrow[b] = a.xq + (long long)min(16 * b + r, a.M - 1) * a.ldq + 16 * g;

  auto load_w = [&](int j, int kk) -> Frag {
    if constexpr (PACKED)
      return load_packed<FMT>(wptr[j], kk);
    else
      return load_frag<FMT>(wptr[j], kk);
  };

  // Block_FP8 scale pointers for this lane: sw row of the 128-row block (the
  // 16*NB rows of a tile never straddle two blocks), and the sx rows of the
  // accumulator elements the lane holds (SWAP: one m per lane; else four).
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
  float ep_sx[MB][SXN], ep_sw[NB][4 / SXN];
  if constexpr (!BLOCK) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < SXN; ++i)
        ep_sx[b][i] = a.sx[min(SWAP ? 16 * b + r : 16 * b + 4 * g + i, a.M - 1)];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4 / SXN; ++i)
        ep_sw[j][i] = a.sw[min(SWAP ? n0 + 16 * j + 4 * g + i : n0 + 16 * j + r, a.N - 1)];
  }

  // K-steps of this split, then of this wave.
  // (32-bit: the host guarantees split_k * ksteps < 2^31.)
  const int ka = (int)((unsigned)(split * a.ksteps) / (unsigned)a.split_k);
  const int kb = (int)((unsigned)((split + 1) * a.ksteps) / (unsigned)a.split_k);
  const int la = ka + (kb - ka) * wk / WK;
  const int lb = ka + (kb - ka) * (wk + 1) / WK;
  const int lfull = min(lb, a.kfull);

  Acc acc[MB][NB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[b][j] = Acc{0, 0, 0, 0};

  // A stage is U consecutive K-steps.  The wave's full K-steps [la, lfull)
  // are covered by ns whole stages ending at lfull; the first stage may
  // start before la, and its steps below la load a clamped (valid) address
  // and are zeroed before their MFMA, so every load of a stage is issued at
  // once and no K-step is ever processed alone.
  struct Stage {
    Frag w[U][NB];
    Frag x[U][MB];
    float sw[BLOCK ? U : 1];
    float sx[BLOCK ? U : 1][MB][SXN];
  };
  auto load_stage = [&](Stage& st, int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = max(k0 + u, la);
#pragma unroll
      for (int j = 0; j < NB; ++j) st.w[u][j] = load_w(j, k);
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
  auto step = [&](const Frag (&w)[NB], const Frag (&x)[MB], float sw, const float (&sx)[MB][SXN]) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        if constexpr (BLOCK) {
          const Acc p = mma<FMT, SWAP>(w[j], x[b], Acc{0, 0, 0, 0});
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[b][j][i] += p[i] * (sx[b][SWAP ? 0 : i] * sw);
        } else {
          acc[b][j] = mma<FMT, SWAP>(w[j], x[b], acc[b][j]);
        }
      }
  };
  // MASK: the first stage, whose steps below la are zeroed.
  auto run_stage = [&](const Stage& st, int k0, auto mask) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Frag w[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const Frag zero = {};
        w[j] = (decltype(mask)::value && k0 + u < la) ? zero : st.w[u][j];
      }
      step(w, st.x[u], st.sw[BLOCK ? u : 0], st.sx[BLOCK ? u : 0]);
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
  // multiple of its 128-byte K-step) belongs to the wave that owns step
  // kfull.  Packed weights are zero-padded there; activations are masked.
  if constexpr (!BLOCK) {
    if (lb > a.kfull && la < lb) {
      Frag wt[NB], xt[MB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        wt[j] = PACKED ? load_w(j, a.kfull) : load_frag_tail<FMT>(wptr[j], a.kfull, 16 * g, a.K);
#pragma unroll
      for (int b = 0; b < MB; ++b) xt[b] = load_frag_tail<FMT>(xrow[b], a.kfull, 16 * g, a.K);
      const float no_sx[MB][SXN] = {};
      step(wt, xt, 0.0f, no_sx);
    }
  }

  // Sum the WK waves through LDS, in wave order.
  if constexpr (WK > 1) {
    __shared__ Acc red[(WK - 1) * MB * NB * 64];
    if (wk > 0) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int j = 0; j < NB; ++j) red[(((wk - 1) * MB + b) * NB + j) * 64 + lane] = acc[b][j];
    }
    __syncthreads();
    if (wk == 0) {
      for (int q = 1; q < WK; ++q)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[b][j] += red[(((q - 1) * MB + b) * NB + j) * 64 + lane];
    }
  }

  // Split-K: publish the partial; the last workgroup of the tile reduces.
  // Protocol (no L2 writeback or invalidate): the partials are written with
  // agent-scope atomic stores, which write through this XCD's L2 to the
  // device-coherent level; s_waitcnt waits until every one of them is
  // acknowledged before the workgroup counts itself in; the last workgroup
  // to arrive reads the partials with agent-scope atomic loads, which are
  // served from the device-coherent level, so it sees every split's data.
  // Partial layout: fragment f = ((tile*S + split)*NB + j)*MB + b holds
  // 4 x 64 words, word (f*4 + i)*64 + lane, so each of the four stores of a
  // wave writes 256 contiguous bytes.
  if (a.split_k > 1) {
    typedef decltype(acc[0][0][0]) Elem;
    typedef typename std::remove_cv<typename std::remove_reference<Elem>::type>::type Word;
    Word* part = reinterpret_cast<Word*>(a.part);
    const long long frag0 = (long long)tile * a.split_k;
    if (wk == 0) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __hip_atomic_store(part + ((((frag0 + split) * NB + j) * MB + b) * 4 + i) * 64 + lane,
                               acc[b][j][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[b][j] = Acc{0, 0, 0, 0};
      for (int s = 0; s < a.split_k; ++s)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[b][j][i] += __hip_atomic_load(
                  part + ((((frag0 + s) * NB + j) * MB + b) * 4 + i) * 64 + lane,
                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (wk != 0) return;

  // Epilogue.
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = SWAP ? 16 * b + r : 16 * b + 4 * g + i;
        const int n = SWAP ? n0 + 16 * j + 4 * g + i : n0 + 16 * j + r;
        if (m < a.M && n < a.N) {
          const long long o = (long long)m * a.ldo + n;
          if (a.out_mode) {
            if constexpr (FMT == W8A8_INT8)
              reinterpret_cast<int*>(a.out)[o] = acc[b][j][i];
            else
              reinterpret_cast<float*>(a.out)[o] = acc[b][j][i];
          } else {
            float y;
            if constexpr (BLOCK) {
              y = acc[b][j][i];
            } else {
              const float sxm = ep_sx[b][SWAP ? 0 : i], swn = ep_sw[j][SWAP ? i : 0];
              if constexpr (FMT == W8A8_INT8)
                y = (float)acc[b][j][i] * sxm * swn;
              else
                y = acc[b][j][i] * sxm * swn;
            }
            reinterpret_cast<uint16_t*>(a.out)[o] = bf16_rne(y);
          }
        }
      }
}

template <int FMT, int MB, int NB, int WK, int U, int SWAP, int PACKED>
hipError_t launch_gemm(const GemmArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<FMT, MB, NB, WK, U, SWAP, PACKED>), grid, block, 0, s, a);
  return hipGetLastError();
}

// Packs row-major codes [N, K] (row stride ldw) into the MFMA-native layout
// (see the kernel header): one thread per 16-byte chunk, zero padding for
// rows >= N and bytes >= K.
template <int KSTEP>
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint8_t* __restrict__ w,
                                                          long long ldw, int N, int K,
                                                          int ksteps, uint8_t* __restrict__ out,
                                                          long long chunks) {
  const long long c = blockIdx.x * 256LL + threadIdx.x;
  if (c >= chunks) return;
  // chunk c: fragment f = c / (KSTEP), within it instruction jj and lane l
  constexpr int CHUNKS_PER_FRAG = 16 * KSTEP / 16;  // = KSTEP
  const long long f = c / CHUNKS_PER_FRAG;
  const int within = (int)(c % CHUNKS_PER_FRAG);
  const int jj = within / 64, l = within % 64;
  const long long nb = f / ksteps;
  const int kk = (int)(f % ksteps);
  const long long row = nb * 16 + (l & 15);
  const long long k = (long long)kk * KSTEP + 64 * jj + 16 * (l >> 4);
  // (K % 16 == 0, so a chunk is either wholly inside K or wholly outside.)
  v4i v = {0, 0, 0, 0};
  if (row < N && k < K) v = *reinterpret_cast<const v4i*>(w + row * ldw + k);
  *reinterpret_cast<v4i*>(out + c * 16) = v;
}

}  // namespace w8
