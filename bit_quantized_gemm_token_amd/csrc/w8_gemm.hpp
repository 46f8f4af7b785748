// The GEMM kernel family: Y[M, N] = dequant(Xq) . dequant(Wq)^T for M <= 32.
//
// ai-radar.it, "Helion nel backend vLLM: un solo GEMM, tuning per forma e
// guadagni fino al 10%", paragraphs 2-3: Standard, Split-K and Swap-AB are
// tunable parameters of one GEMM implementation; split_k is a power of two up
// to 256; the search also covers memory layout.  Here they are template and
// launch parameters of one kernel:
//
//   wave   owns NB blocks of 16 weight rows; a workgroup has WK x WN waves:
//          WK waves split the workgroup's K range (summed through LDS in
//          wave order), WN waves sit side by side along N (tile = WN*NB row
//          blocks) and share the activations staged in LDS (one of WK, WN is
//          1; WN > 1 needs XL).
//   grid   grid == 0: ntiles * split_k workgroups, one per (tile, split), the
//          split index varying fastest.  Workgroups are dealt round-robin to
//          the 8 XCDs, each with its own L2, so with split_k a power of two
//          an XCD sees only split_k/8 K ranges (split_k >= 8) or one (split_k
//          < 8), and fetches only those activation columns instead of all K.
//          grid > 0 (stream-K, instances compiled with SK = 1): exactly
//          `grid` workgroups share the ntiles x ksteps (tile, K-step)
//          iterations in equal contiguous ranges, so the weight stream is
//          spread evenly over the compute units whatever the tile count; a
//          tile split between workgroups is summed like a split-K tile.  The
//          split-K instances (SK = 0) carry none of its code: its loop and
//          64-bit range arithmetic would cost the common path registers.
//   K loop one MFMA per K-step, row block and 16-row block of M (64 bytes of K
//          for int8, 128 for E4M3FN); each lane streams its weight bytes
//          straight from HBM into MFMA operand registers with 16-byte loads
//          (no LDS for weights: every weight byte meets at most 32 tokens, so
//          there is nothing to reuse), U K-steps per stage, two stages in
//          flight.  XL == 0: the wave loads its own activation fragments in
//          each stage (reused by its NB row blocks).  XL == 1: before the K
//          loop the workgroup copies the activation fragments of its K range
//          into LDS with direct-to-LDS loads, each wave a share of them, and
//          the K loop reads them from LDS: the loop's vector-memory pipe then
//          carries only weights, and with WN > 1 every activation byte is
//          fetched once per workgroup instead of once per wave.  (A compute
//          unit moves about 20 bytes per clock through its vector-memory
//          path whether a load hits or misses; at M = 32 the activation
//          fragments are as many bytes as the weights.)
//   layout PACKED=0: Wq row-major [N, K] (row stride ldw); a load instruction
//          reads 64 contiguous bytes of 16 rows.  PACKED=1: the MFMA-native
//          layout written by the weight packer: the 16 x KSTEP bytes of one
//          (row block, K-step) fragment are stored in lane order, so every
//          load instruction reads 1 KiB contiguous and a wave's whole K range
//          is one contiguous run; rows and K are zero-padded to whole
//          fragments.  Packed loads are non-temporal (each line is read once).
//   K-segmented layouts PACKED = T in {2, 4, 8}: one MFMA takes R = 16/T
//          weight rows times T consecutive K-steps (a "span"): operand index
//          p = lane % 16 is split as p = t*R + r (K-step t of the span, row
//          r), and the activation operand likewise as p = t*R + m (token m
//          of a group of R tokens).  Of the 16 x 16 products only the blocks
//          with equal t are wanted; they are summed over t at the end.  A
//          fragment (R rows, one span) is again 16 x KSTEP bytes in lane
//          order, so the loads are as contiguous as with PACKED=1, but a row
//          block is R rows instead of 16: at M <= R tokens the same weight
//          bytes make 16/R times as many output tiles, which spreads a
//          narrow N over the compute units without splitting K (and without
//          the split-K hand-off).  The K loop runs over spans; a span that
//          reaches past K is masked like the ragged K-step.
//   Swap-AB SWAP=0: A = activations, B = weights^T, C[m][n];
//          SWAP=1: A = weights, B = activations^T, C[n][m] = (Wq . Xq^T)^T.
//          The MFMA work is identical (square 16x16 tiles); what changes is
//          the accumulator-to-lane map and so the epilogue's store pattern.
//   Split-K / shared tiles  each contributing workgroup writes its partial
//          tile to the workspace; the last one of the tile to arrive (arrival
//          counter) sums the partials in K order and runs the epilogue.  The fixed order makes results run-to-run
//          deterministic; empty splits (split_k > number of K-steps)
//          contribute zeros.
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

// Phase stamps, for timing studies only: unless W8_PHASE_STAMPS is defined
// (the library never defines it; csrc/w8_phase_probe.hip does) they compile
// to nothing.  Defined, thread 0 of each workgroup -- and lane 0 of each
// wave for the end of its K loop -- records s_memrealtime (a 100 MHz
// counter common to the whole device) into a record of 32 words per
// workgroup that starts W8_PHASE_STAMPS bytes past the output: word 0 the
// segment's start, 1 wave 0's K loop done, 2 the K-waves summed, 3 the
// partials acknowledged, 4 the arrival count returned, 6 the output stored
// (the workgroup that owns its tile or is the last to arrive), 7 done
// without storing, 8 + w the end of wave w's K loop.  Words 6 and 7 are
// taken after the stores and loads in flight have completed.
#ifdef W8_PHASE_STAMPS
#define W8_STAMP_AT(slot)                                                              \
  do {                                                                                 \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                                           \
    reinterpret_cast<unsigned long long*>(static_cast<char*>(a.out) +                  \
                                          W8_PHASE_STAMPS)[blockIdx.x * 32 + (slot)] = \
        __builtin_amdgcn_s_memrealtime();                                              \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                                           \
  } while (0)
#define W8_STAMP(i)                        \
  do {                                     \
    if (threadIdx.x == 0) W8_STAMP_AT(i); \
  } while (0)
#define W8_STAMP_DONE(i)                 \
  do {                                   \
    __builtin_amdgcn_s_waitcnt(0);       \
    W8_STAMP(i);                         \
  } while (0)
#define W8_STAMP_WAVE()                                                   \
  do {                                                                    \
    if ((threadIdx.x & 63) == 0) W8_STAMP_AT(8 + (int)(threadIdx.x >> 6)); \
  } while (0)
#else
#define W8_STAMP(i) \
  do {              \
  } while (0)
#define W8_STAMP_DONE(i) \
  do {                   \
  } while (0)
#define W8_STAMP_WAVE() \
  do {                  \
  } while (0)
#endif

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

// The body of one GEMM workgroup.  GROUPED (the MoE grouped GEMM): activation
// row m of this call is row xrows[m] (clamped to [0, xrow_max]) of the
// activation codes and scales (XL == 2: of the bf16 activations); everything
// else is per call in `a`.
template <int FMT, int MB, int NB, int WK, int WN, int U, int SWAP, int PACKED, int XL, int SK,
          bool GROUPED>
__device__ __forceinline__ void gemm_body(GemmArgs a, const int* __restrict__ xrows,
                                          int xrow_max) {
  typedef typename Traits<FMT>::Frag Frag;
  typedef typename Traits<FMT>::Acc Acc;
  constexpr int KSTEP = Traits<FMT>::KSTEP;
  constexpr bool BLOCK = (FMT == BLOCK_FP8);
  static_assert(WN == 1 || WK == 1, "the waves of a workgroup split either K or N");
  static_assert(WN == 1 || XL, "waves side by side along N share activations through LDS");
  static_assert(XL != 3 || (BLOCK && WN == 1), "quantization in the K loop: Block_FP8, WN == 1");
  // K-segmented layouts: T K-steps per MFMA, row blocks of R = 16/T weight
  // rows, token groups of R rows (T = 1: the plain 16 x 16 tile).
  constexpr int T = PACKED > 1 ? PACKED : 1;
  constexpr int R = 16 / T;
  static_assert(T == 1 || T == 2 || T == 4 || T == 8, "segments per MFMA: 1, 2, 4 or 8");
  static_assert(T == 1 || ((XL == 0 || XL == 2) && WN == 1 && SK == 0 && !GROUPED),
                "K-segmented layouts: plain activation loads or fused quantization, one wave "
                "along N, split-K only");
  // activation row (codes and scales, or XL == 2 the bf16 row) of row m of
  // this call
  auto xr = [&](int m) -> long long {
    if constexpr (GROUPED)
      return min(max(xrows[m], 0), xrow_max);
    else
      return m;
  };
  // XL 3 (Block_FP8 linear): no staging; each wave loads the bf16
  // activations of its K-steps in its stages and quantizes every 1x128
  // group in the K loop.  (Not for the per-token formats: a wave quantizes
  // all 16 rows of its MFMA tile at every K-step whatever M is, and every
  // workgroup repeats it, so the quantization's ALU work outweighs the
  // separate launch it saves -- measured 3-4x slower.)
  // XL 1, 2: the segment's activation fragments are staged in LDS up front, one
  // 1 KiB chunk (16 bytes per lane) per (K-step, M block, 16-byte load):
  // chunk ((k - ka) * MB + b) * CH + jj.  XL == 1 copies the codes; XL == 2
  // (fused quantization) quantizes bf16 activations into them.
  constexpr int CH = KSTEP / 64;
  constexpr bool INT8 = (FMT == W8A8_INT8);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wk = wave % WK, wn = wave / WK;
  const int r = lane & 15, g = lane >> 4;
  // The lane's operand index r = tl*R + mr: K-step tl of the span and row mr
  // of its block (T = 1: tl = 0, mr = r).
  const int tl = r / R, mr = r % R;

  // Activation rows of this lane (padding rows of the MFMA tile read a
  // clamped valid row; their outputs are never stored).
  const uint8_t* xrow[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
    xrow[b] = a.xq + xr(min(R * b + mr, a.M - 1)) * a.ldq + tl * KSTEP + 16 * g;
  // XL == 3: the lane's bf16 activations (row stride ldq in elements), the
  // same 2 x 16 elements of each K-step whose codes it feeds to the MFMA.
  const uint16_t* xrow16[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
    xrow16[b] = reinterpret_cast<const uint16_t*>(a.xq) + xr(min(16 * b + r, a.M - 1)) * a.ldq +
                16 * g;

  // Block_FP8 sx rows of the accumulator elements this lane holds (SWAP: one
  // m per lane; else four); the per-token formats' epilogue sx are loaded in
  // the segment, after its first weight stages (see there).
  constexpr int SXN = SWAP ? 1 : 4;
  const int nthreads = 64 * WK * WN;
  __shared__ Acc red[WK > 1 ? (WK - 1) * MB * NB * 64 : 1];
  __shared__ v4i xl[(XL == 1 || XL == 2) ? kXlChunks * 64 : 1];
  // XL == 1, Block_FP8: the segment's activation scales, group-major
  // (entry kk * 16 * MB + row for K-step ka + kk), staged with the codes
  // (at most kXlChunks / 2 K-steps of 32 rows, plus a partial last copy).
  __shared__ float sxs[(XL == 1 && BLOCK) ? kXlMaxGroups * 32 + 64 : 1];
  // XL == 2: activation scales computed here -- per row for the per-token
  // formats, per (staged group, row) for Block_FP8.
  __shared__ float sxl[XL == 2 ? (BLOCK ? kXlMaxGroups * 32 : 32) : 1];
  __shared__ int is_last;
  // K-segmented layouts: the wave's accumulator tiles for the epilogue's
  // sums over t (WN == 1: one region).
  __shared__ Acc dgl[T > 1 ? NB * MB * 64 : 1];

  if constexpr (XL == 2 && !BLOCK) {
    // Row absolute maxima (float bits), folded in by the first segment.
    if (threadIdx.x < 32) reinterpret_cast<unsigned*>(sxl)[threadIdx.x] = 0u;
    __syncthreads();
  }
  bool rows_done = false;  // XL == 2, per-token formats: row scales computed

  const float* sxrow[MB][SXN];
  int sxm[MB][SXN];  // row of each accumulator element this lane holds (clamped)
  float ep_sx[MB][SXN];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < SXN; ++i) {
      const int m = min(SWAP ? R * b + mr : R * b + (4 * g + i) % R, a.M - 1);
      sxm[b][i] = m;
      if constexpr (BLOCK) {
        sxrow[b][i] = XL >= 2 ? nullptr : a.sx + xr(m) * a.sgroups;
        ep_sx[b][i] = 0.0f;
      } else {
        sxrow[b][i] = nullptr;
        ep_sx[b][i] = 0.0f;  // loaded in the segment, or (XL == 2) computed by the row pass
      }
    }

  // Per-token formats, XL == 2: row absolute maxima over the whole of K.
  // Each row is split over max(1, waves / M) waves, each lane keeps a
  // running maximum of its chunks (two or four loads in flight), one wave
  // reduction per (row, part), folded into the row's word (|x| >= 0: its
  // float bits order as unsigned integers); then the epilogue's row scales.
  auto row_pass = [&]() {
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.xq);
    unsigned* amx = reinterpret_cast<unsigned*>(sxl);
    const int nw = WK * WN;
    const int wpr = max(1, nw / a.M);  // waves per row
    const int cpr = a.K / 8;           // 16-byte chunks per row
    const int step = 64 * wpr;
    for (int slot = wave; slot < a.M * wpr; slot += nw) {
      const int m = slot / wpr, part = slot - m * wpr;
      const uint16_t* rowp = xb + xr(m) * a.ldq;
      float mx = 0.0f;
      constexpr int QA = WK * WN >= 8 ? 2 : 4;  // loads in flight per lane (registers)
      for (int c0 = part * 64 + lane; c0 < cpr; c0 += QA * step) {
        v4u v[QA];
#pragma unroll
        for (int q = 0; q < QA; ++q) {
          const int c = c0 + q * step;
          v[q] = v4u{0u, 0u, 0u, 0u};
          if (c < cpr) v[q] = *reinterpret_cast<const v4u*>(rowp + 8 * c);
        }
#pragma unroll
        for (int q = 0; q < QA; ++q) mx = fmaxf(mx, absmax8(v[q]));
      }
      mx = wave_max(mx);
      if (lane == 0) atomicMax(&amx[m], __float_as_uint(mx));
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < SXN; ++i) ep_sx[b][i] = act_scale<INT8>(__uint_as_float(amx[sxm[b][i]]));
    rows_done = true;
  };

  // K-segmented layouts: the wave's NB x MB blocks give NB*MB*R*R outputs,
  // dealt to the lanes OPL at a time in the epilogue: output o = lane + 64q
  // is (block j, token group b, token m, row rr) with rr varying fastest, so
  // neighbouring lanes store neighbouring columns of Y.
  constexpr int NOUT = NB * MB * R * R;
  constexpr int OPL = T > 1 ? (NOUT + 63) / 64 : 1;

  // One segment: K-steps [ka, kb) (spans for the K-segmented layouts) of
  // output tile `tile` (WN*NB blocks of 16, or R, weight rows).  The segment
  // is contributor `slot` of the `count` workgroups that cover the tile;
  // count == 1 writes Y directly.
  auto segment = [&](int tile, int ka, int kb, int slot, int count) {
    W8_STAMP(0);
    const int n0 = (tile * WN + wn) * R * NB;  // first weight row of this wave

    const uint8_t* wptr[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (PACKED) {
        const int nb = min((tile * WN + wn) * NB + j, (a.N + R - 1) / R - 1);
        wptr[j] = a.wq + (long long)nb * a.ksteps * (16 * KSTEP) + 16 * lane;
      } else {
        wptr[j] = a.wq + (long long)min(n0 + 16 * j + r, a.N - 1) * a.ldw + 16 * g;
      }
    }
    auto load_w = [&](int j, int kk) -> Frag {
      if constexpr (PACKED)
        return load_packed<FMT>(wptr[j], kk);
      else
        return load_frag<FMT>(wptr[j], kk);
    };
    // Block_FP8 sw row of the wave's 128-row block (its R*NB rows never
    // straddle two blocks); the per-token formats' epilogue sw.
    const float* swrow = nullptr;
    float ep_sw[NB][4 / SXN];
    float ep2_sw[OPL], ep2_sx[OPL];  // K-segmented layouts: per output of the lane
    if constexpr (BLOCK) swrow = a.sw + (long long)(min(n0, a.N - 1) / kGroup) * a.sgroups;
    // The per-token formats' epilogue scales, issued after the first weight
    // stages: vector-memory loads complete in issue order, so a scale load
    // issued first would hold up the first MFMA behind its own latency.
    auto load_epilogue_scales = [&]() {
      if constexpr (!BLOCK && T > 1) {
#pragma unroll
        for (int q = 0; q < OPL; ++q) {
          const int o = min(lane + 64 * q, NOUT - 1);
          const int jb = o / (R * R), m = (o / R) % R, rr = o % R;
          ep2_sw[q] = a.sw[min(n0 + R * (jb / MB) + rr, a.N - 1)];
          // (XL == 2: the row scales are computed by the row pass instead)
          if constexpr (XL != 2) ep2_sx[q] = a.sx[xr(min(R * (jb % MB) + m, a.M - 1))];
        }
      } else if constexpr (!BLOCK) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int i = 0; i < 4 / SXN; ++i)
            ep_sw[j][i] = a.sw[min(SWAP ? n0 + 16 * j + 4 * g + i : n0 + 16 * j + r, a.N - 1)];
        if constexpr (XL != 2) {
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int i = 0; i < SXN; ++i) ep_sx[b][i] = a.sx[xr(sxm[b][i])];
        }
      }
    };

    // K-steps of this wave: its WK-th of the segment.
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
    // and are zeroed before their MFMA, so every load of a stage is issued
    // at once and no K-step is ever processed alone.
    struct Stage {
      Frag w[U][NB];
      Frag x[XL ? 1 : U][MB];  // !XL: the wave's own activation fragments
      v4u xb[XL == 3 ? U : 1][XL == 3 ? MB : 1][CH][2];  // XL == 3: bf16, quantized in run_stage
      // Block_FP8 scales of each K-step: the weight scale, and for XL == 0
      // the activation scale of each accumulator row (XL == 1 stages them in
      // LDS with the codes, XL >= 2 computes them in the kernel).
      float sw[BLOCK ? U : 1];
      float sx[BLOCK && XL == 0 ? U : 1][MB][SXN];
    };
    auto load_stage = [&](Stage& st, int k0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = max(k0 + u, la);
#pragma unroll
        for (int j = 0; j < NB; ++j) st.w[u][j] = load_w(j, k);
        if constexpr (!XL) {  // (K-segmented: span k starts at K-step k*T)
#pragma unroll
          for (int b = 0; b < MB; ++b) st.x[u][b] = load_frag<FMT>(xrow[b], k * T);
        }
        if constexpr (XL == 3) {
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int jj = 0; jj < CH; ++jj) {
              const uint16_t* src = xrow16[b] + (long long)k * KSTEP + 64 * jj;
              st.xb[u][b][jj][0] = *reinterpret_cast<const v4u*>(src);
              st.xb[u][b][jj][1] = *reinterpret_cast<const v4u*>(src + 8);
            }
        }
        if constexpr (BLOCK) {
          // group of the lane's own K-step (K-segmented: the group of the
          // products the lane keeps, K-step k*T + tl)
          const int kg = k * T + tl;
          if constexpr (T == 1) {
            // one value for the whole wave (its rows lie in one 128-row
            // block): a scalar load, off the vector-memory path
            st.sw[u] = *(const __attribute__((address_space(4))) float*)(swrow + kg);
          } else {
            st.sw[u] = swrow[kg];
          }
          if constexpr (XL == 0) {
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
              for (int i = 0; i < SXN; ++i) st.sx[u][b][i] = sxrow[b][i][kg];
          }
        }
      }
    };

    // sc: Block_FP8's sx * sw of each accumulator element (ignored otherwise)
    auto step = [&](const Frag (&w)[NB], const Frag (&x)[MB], const float (&sc)[MB][SXN]) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          if constexpr (BLOCK) {
            const Acc p = mma<FMT, SWAP>(w[j], x[b], Acc{0, 0, 0, 0});
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[b][j][i] += p[i] * sc[b][SWAP ? 0 : i];
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
        if constexpr (XL == 3) {
          // Quantize the loaded 1x128 groups (the standalone quantizer's
          // steps): the four lanes l, l^16, l^32, l^48 hold one row's group,
          // so two shuffles give its maximum; SWAP = 0 accumulator lanes get
          // their rows' scales from lane 4g + i.
          Frag x[MB];
          float sx[MB][SXN];
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            float gm = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
              gm = fmaxf(gm, fmaxf(absmax8(st.xb[u][b][jj][0]), absmax8(st.xb[u][b][jj][1])));
            gm = fmaxf(gm, __shfl_xor(gm, 16, 64));
            gm = fmaxf(gm, __shfl_xor(gm, 32, 64));
            const float sc = act_scale<false>(gm);
            const float rs = act_recip(sc);
            v4i q[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const v2u ql = encode8<false>(st.xb[u][b][jj][0], sc, rs),
                        qh = encode8<false>(st.xb[u][b][jj][1], sc, rs);
              q[jj] = v4i{(int)ql[0], (int)ql[1], (int)qh[0], (int)qh[1]};
            }
            x[b] = __builtin_shufflevector(q[0], q[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int i = 0; i < SXN; ++i)
              sx[b][i] = (SWAP ? sc : __shfl(sc, 4 * g + i, 64)) * st.sw[u];
          }
          step(w, x, sx);
        } else if constexpr (XL) {
          const int k = max(k0 + u, la);
          Frag x[MB];
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            const int c = ((k - ka) * MB + b) * CH;
            if constexpr (FMT == W8A8_INT8) {
              x[b] = xl[c * 64 + lane];
            } else {
              const v4i lo = xl[c * 64 + lane];
              const v4i hi = xl[(c + 1) * 64 + lane];
              x[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
          }
          float sc[MB][SXN] = {};
          if constexpr (XL == 2 && BLOCK) {
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
              for (int i = 0; i < SXN; ++i)
                sc[b][i] =
                    sxl[((k - ka) * MB + b) * 16 + (SWAP ? r : tl * R + (4 * g + i) % R)] * st.sw[u];
          } else if constexpr (BLOCK) {  // XL == 1 (T == 1): the staged scales
#pragma unroll
            for (int b = 0; b < MB; ++b) {
              const int e = (k - ka) * 16 * MB + 16 * b;
              if constexpr (SWAP) {
                sc[b][0] = sxs[e + r] * st.sw[u];
              } else {
                const v4f v = *reinterpret_cast<const v4f*>(&sxs[e + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[b][i] = v[i] * st.sw[u];
              }
            }
          }
          step(w, x, sc);
        } else {
          float sc[MB][SXN] = {};
          if constexpr (BLOCK) {
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
              for (int i = 0; i < SXN; ++i) sc[b][i] = st.sx[u][b][i] * st.sw[u];
          }
          step(w, st.x[u], sc);
        }
      }
    };
    const std::true_type masked;
    const std::false_type whole;

    // XL == 1: every wave of the workgroup copies its share of the segment's
    // full K-steps [ka, min(kb, kfull)) of activations into LDS with
    // direct-to-LDS loads (no registers), issued before the weight loads.
    if constexpr (XL == 1) {
      const int nchunks = (min(kb, a.kfull) - ka) * MB * CH;
      for (int c = wave; c < nchunks; c += WK * WN) {
        const int kk = c / (MB * CH), b = (c / CH) % MB, jj = c % CH;
        const uint8_t* src = a.xq + xr(min(16 * b + r, a.M - 1)) * a.ldq + 16 * g +
                             (long long)(ka + kk) * KSTEP + 64 * jj;
        __builtin_amdgcn_global_load_lds(
            src, (__attribute__((address_space(3))) void*)(xl + c * 64), 16, 0, 0);
      }
      if constexpr (BLOCK) {
        // and the scales of the segment's rows and groups, 64 a load
        // (Block_FP8: K % 128 == 0, so every K-step is whole; the entries
        // past the end of the last copy reread the last one)
        const int nsx = (kb - ka) * 16 * MB;
        for (int c = wave * 64; c < nsx; c += 64 * WK * WN) {
          const int e = min(c + lane, nsx - 1);
          const int kk = e / (16 * MB), row = e % (16 * MB);
          const float* src = a.sx + xr(min(row, a.M - 1)) * a.sgroups + ka + kk;
          __builtin_amdgcn_global_load_lds(
              src, (__attribute__((address_space(3))) void*)(sxs + c), 4, 0, 0);
        }
      }
    }

    // Stages alternate between register sets A and B: the loads of stage s+1
    // are issued before stage s feeds the MFMAs.
    const int ns = (max(lfull - la, 0) + U - 1) / U;
    const int k0 = lfull - ns * U;
    Stage A, B;
    if (ns > 0) load_stage(A, k0);
    if (ns > 1) load_stage(B, k0 + U);
    load_epilogue_scales();
    // XL == 2: quantize the segment's activations into the LDS stage.  The
    // raw bf16 slice is fetched while the first weight stages are in flight
    // (and, for the per-token formats, together with the row pass), so one
    // memory latency covers all of them.  Scales and codes follow the
    // standalone quantizer (per-token formats: the row's absolute maximum
    // over the whole of K, computed in the first segment; Block_FP8: each
    // staged 1x128 group), with the same encoder, so the codes equal its
    // codes byte for byte.  A unit is (K-step, row block, lane): the CH
    // 16-byte chunks lane l of that MFMA operand reads; a wave's 64 units
    // share one K-step and row block, so the four lanes l, l^16, l^32, l^48
    // hold one row's whole K-step, a Block_FP8 group.  The ragged K tail step
    // is staged too, its bytes past K as zero codes.  (K-segmented layouts:
    // a unit is (span, token group, lane), lane l holding row (l%16)%R of the
    // group at K-step (l%16)/R of the span; the four lanes still share one
    // row's K-step.)  Block_FP8 group scales go to sxl[(kk*MB + b)*16 + p]
    // for the unit's K-step kk of the segment, group b and operand index p.
    if constexpr (XL == 2) {
      const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.xq);
      constexpr int QB = WK * WN >= 8 ? 1 : 2;  // units per thread per batch (registers)
      const int nunits = (kb - ka) * MB * 64;
      v4u raw[QB][CH][2];
      auto fetch = [&](int u0) {
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const int u = u0 + q * nthreads;
          const int kk = u / (MB * 64), b = (u >> 6) % MB;
          const int row = min(R * b + mr, a.M - 1);
#pragma unroll
          for (int jj = 0; jj < CH; ++jj) {
            // first element
            const int e = ((ka + kk) * T + tl) * KSTEP + 64 * jj + 16 * (lane >> 4);
            raw[q][jj][0] = raw[q][jj][1] = v4u{0u, 0u, 0u, 0u};
            if (u < nunits && e < a.K) {  // (K % 16 == 0: a chunk is wholly inside K or past it)
              const uint16_t* src = xb + xr(row) * a.ldq + e;
              raw[q][jj][0] = *reinterpret_cast<const v4u*>(src);
              raw[q][jj][1] = *reinterpret_cast<const v4u*>(src + 8);
            }
          }
        }
      };
      auto put = [&](int u0) {
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const int u = u0 + q * nthreads;  // wave-uniform validity (nunits % 64 == 0)
          const int kk = u / (MB * 64), b = (u >> 6) % MB;
          const int row = min(R * b + mr, a.M - 1);
          float s;
          if constexpr (BLOCK) {
            float gm = 0.0f;
#pragma unroll
            for (int jj = 0; jj < CH; ++jj)
              gm = fmaxf(gm, fmaxf(absmax8(raw[q][jj][0]), absmax8(raw[q][jj][1])));
            gm = fmaxf(gm, __shfl_xor(gm, 16, 64));
            gm = fmaxf(gm, __shfl_xor(gm, 32, 64));
            s = act_scale<false>(gm);
            if (u < nunits && lane < 16) sxl[(kk * MB + b) * 16 + lane] = s;
          } else {
            s = act_scale<INT8>(__uint_as_float(reinterpret_cast<const unsigned*>(sxl)[row]));
          }
          if (u < nunits) {
            const float rs = act_recip(s);
#pragma unroll
            for (int jj = 0; jj < CH; ++jj) {
              const v2u ql = encode8<INT8>(raw[q][jj][0], s, rs),
                        qh = encode8<INT8>(raw[q][jj][1], s, rs);
              xl[((kk * MB + b) * CH + jj) * 64 + lane] =
                  v4i{(int)ql[0], (int)ql[1], (int)qh[0], (int)qh[1]};
            }
          }
        }
      };
      fetch(threadIdx.x);
      if constexpr (!BLOCK) {
        if (!rows_done) row_pass();
      }
      put(threadIdx.x);
      for (int u0 = threadIdx.x + QB * nthreads; u0 < nunits; u0 += QB * nthreads) {
        fetch(u0);
        put(u0);
      }
    }
    if constexpr (XL == 1 || XL == 2) {
      // the copies (and the first weight stages) have landed in every wave
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (ns == 1) {
      run_stage(A, k0, masked);
    } else if (ns > 1) {
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
    W8_STAMP(1);
    W8_STAMP_WAVE();
    // The ragged K tail (K % KSTEP != 0; for the K-segmented layouts, a
    // span reaching past K) belongs to the wave that owns step (span) kfull.
    // Packed weights are zero-padded there; activations are masked by byte.
    // (Block_FP8's K is a multiple of its 128-byte K-step: only a span can
    // reach past K; its groups past K have zero codes, and their scale reads
    // are clamped to the last group.)
    if constexpr (!BLOCK || T > 1) {
      if (lb > a.kfull && la < lb) {
        Frag wt[NB], xt[MB];
        float tsw = 0.0f, tsx[MB][SXN] = {};
        if constexpr (BLOCK) {
          const int kg = min(a.kfull * T + tl, a.sgroups - 1);
          tsw = swrow[kg];
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int i = 0; i < SXN; ++i) {
              if constexpr (XL == 2)  // the staged span's group scales
                tsx[b][i] = sxl[((a.kfull - ka) * MB + b) * 16 +
                                (SWAP ? r : tl * R + (4 * g + i) % R)];
              else
                tsx[b][i] = sxrow[b][i][kg];
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j)
          wt[j] = PACKED ? load_w(j, a.kfull) : load_frag_tail<FMT>(wptr[j], a.kfull, 16 * g, a.K);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          if constexpr (XL == 2) {
            const int c = ((a.kfull - ka) * MB + b) * CH;  // staged, zero past K
            if constexpr (FMT == W8A8_INT8) {
              xt[b] = xl[c * 64 + lane];
            } else {
              const v4i lo = xl[c * 64 + lane];
              const v4i hi = xl[(c + 1) * 64 + lane];
              xt[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
          } else {
            xt[b] = load_frag_tail<FMT>(xrow[b], a.kfull * T, tl * KSTEP + 16 * g, a.K);
          }
        }
        float tsc[MB][SXN];
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int i = 0; i < SXN; ++i) tsc[b][i] = tsx[b][i] * tsw;
        step(wt, xt, tsc);
      }
    }

    // Sum the WK waves through LDS, in wave order.
    if constexpr (WK > 1) {
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

    W8_STAMP(2);
    // Several workgroups cover this tile: publish the partial; the last
    // workgroup to arrive sums them in slot (= K) order.
    // Protocol (no L2 writeback or invalidate): the partials are written with
    // agent-scope (SC1) stores, which write through this XCD's L2 to the
    // device-coherent level; s_waitcnt waits until every one of them is
    // acknowledged before the workgroup counts itself in; the last workgroup
    // to arrive reads the partials with agent-scope (SC1) loads, which are
    // served from the device-coherent level, so it sees every slot's data.
    // (An agent-scope release on the count and acquire in the last arriver
    // would write back and invalidate whole L2s: measured 1.5 to 9 us more
    // per launch.)  Partial layout: the tile's slots * WN * NB * MB fragments
    // of 1 KiB, fragment ((slot * WN + wn) * NB + j) * MB + b holding lane
    // l's four accumulator words at 16 l, so one store or load instruction
    // of a wave moves 1 KiB contiguous.
    bool store = true;
    if (count > 1) {
      // fragments per tile: slots <= 256 (split-K) or <= K-steps <= 2^16
      // (stream-K, WN * NB * MB <= 16 there), so byte offsets fit in 31 bits
      const int tfrags = a.slots * WN * NB * MB;
      const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(
          static_cast<char*>(a.part) + (long long)tile * tfrags * 1024, tfrags * 1024);
      auto foff = [&](int sl, int j, int b) {
        return (((sl * WN + wn) * NB + j) * MB + b) * 1024 + 16 * lane;
      };
      if (wk == 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int b = 0; b < MB; ++b)
            coherent_store16(prs, foff(slot, j, b), __builtin_bit_cast(v4i, acc[b][j]));
      }
      // The compiler may not move memory operations across the wait (the
      // signal fences); the hardware keeps the order: s_waitcnt vmcnt(0)
      // returns only when every store above has been acknowledged by the
      // level it was written through to, and the count is issued after it.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __syncthreads();
      W8_STAMP(3);
      // Arrival counting.  Split-K (count = split_k, a power of two <= 256):
      // each contributor adds 256 / count to word 0 of the tile's counter
      // line, so a launch raises it by exactly 256 and the counter is never
      // reset (it stays a multiple of 256 between launches; a zero-filled
      // workspace starts it so); the contributor that completes a multiple
      // of 256 is the last.  Stream-K (any count): word 1 counts from zero
      // and the last contributor resets it.
      unsigned* ctr = a.counters + (long long)tile * kCounterWords + (SK ? 1 : 0);
      if (threadIdx.x == 0) {
        const unsigned inc = SK ? 1u : 256u / (unsigned)count;
        const unsigned prev =
            __hip_atomic_fetch_add(ctr, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = SK ? prev == (unsigned)(count - 1) : ((prev + inc) & 255u) == 0u;
      }
      __syncthreads();
      store = is_last;
      W8_STAMP(4);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the partial loads stay after the count
      if (store) {
        if (wk == 0) {
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[b][j] = Acc{0, 0, 0, 0};
          // Slots are read in batches of up to Q (at most 16 fragments, all
          // loads of a batch in flight at once), then added in slot order.
          constexpr int Q = (NB * MB >= 16) ? 1 : 16 / (NB * MB);
          for (int s0 = 0; s0 < count; s0 += Q) {
            v4i v[Q][NB][MB];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
              if (s0 + q < count) {  // (wave-uniform)
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                  for (int b = 0; b < MB; ++b) v[q][j][b] = coherent_load16(prs, foff(s0 + q, j, b));
              }
            }
#pragma unroll
            for (int q = 0; q < Q; ++q) {
              if (s0 + q < count) {
#pragma unroll
                for (int j = 0; j < NB; ++j)
#pragma unroll
                  for (int b = 0; b < MB; ++b) acc[b][j] += __builtin_bit_cast(Acc, v[q][j][b]);
              }
            }
          }
        }
        if (SK && threadIdx.x == 0)
          __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (!store || wk != 0) {
      if (!store) W8_STAMP_DONE(7);
      return;
    }

    if constexpr (T > 1) {
      // K-segmented epilogue: the wave writes its 16 x 16 tiles to LDS as
      // [block][column][row] and each output sums its T wanted products in
      // t order: SWAP = 1, rows are weight rows (t, rr), columns tokens
      // (t, m); SWAP = 0 the other way round.  (The LDS region is the
      // wave's own and a wave's LDS accesses complete in order; the signal
      // fences keep the compiler from moving the reads above the writes.)
      typedef decltype(acc[0][0][0]) Elem;
      typedef typename std::remove_cv<typename std::remove_reference<Elem>::type>::type Word;
      Word* d = reinterpret_cast<Word*>(dgl);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
          *reinterpret_cast<Acc*>(d + ((j * MB + b) * 16 + r) * 16 + 4 * g) = acc[b][j];
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      // Every value first, then the stores (see the plain epilogue below).
      Word vv[OPL];
      uint16_t yb[OPL];
#pragma unroll
      for (int q = 0; q < OPL; ++q) {
        const int o = min(lane + 64 * q, NOUT - 1);
        const int jb = o / (R * R), m = (o / R) % R, rr = o % R;
        Word v = 0;
#pragma unroll
        for (int t = 0; t < T; ++t)
          v += SWAP ? d[(jb * 16 + t * R + m) * 16 + t * R + rr]
                    : d[(jb * 16 + t * R + rr) * 16 + t * R + m];
        vv[q] = v;
        float y;
        if constexpr (BLOCK) {
          y = v;
        } else {
          float sxv;
          if constexpr (XL == 2)  // from the row pass's absolute maximum of row mm
            sxv = act_scale<INT8>(__uint_as_float(
                reinterpret_cast<const unsigned*>(sxl)[min(R * (jb % MB) + m, a.M - 1)]));
          else
            sxv = ep2_sx[q];
          y = (float)v * sxv * ep2_sw[q];
        }
        yb[q] = bf16_rne(y);
      }
      __builtin_amdgcn_s_waitcnt(0);  // (see the plain epilogue below)
#pragma unroll
      for (int q = 0; q < OPL; ++q) {
        const int o = lane + 64 * q;
        const int jb = o / (R * R), m = (o / R) % R, rr = o % R;
        const int mm = R * (jb % MB) + m, n = n0 + R * (jb / MB) + rr;
        if (o < NOUT && mm < a.M && n < a.N) {
          const long long off = (long long)mm * a.ldo + n;
          if (a.out_mode)
            reinterpret_cast<Word*>(a.out)[off] = vv[q];
          else
            reinterpret_cast<uint16_t*>(a.out)[off] = yb[q];
        }
      }
      W8_STAMP_DONE(6);
      return;
    }

    // Epilogue: every value first, then one wait for all outstanding loads,
    // then the stores.  (Without the explicit wait the compiler re-waited
    // vmcnt(0) at the top of every guarded store: a lane-empty branch may
    // skip a block, so at each join it still counts earlier loads as
    // pending, and on gfx9 vmcnt(0) also waits for the stores issued
    // before -- the stores went out one at a time, ~0.6 us for eight.)
    uint16_t yb[MB][NB][4];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
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
          yb[b][j][i] = bf16_rne(y);
        }
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // MFMA 16x16 C layout: lane holds column lane%16, rows 4*(lane/16)+i.
          // SWAP=0: C[m][n]: m = 16b + 4g + i, n = n0 + 16j + r.
          // SWAP=1: C[n][m]: n = n0 + 16j + 4g + i, m = 16b + r.
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
              reinterpret_cast<uint16_t*>(a.out)[o] = yb[b][j][i];
            }
          }
        }
    W8_STAMP_DONE(6);
  };

  if constexpr (!SK) {
    // One workgroup per (tile, split); the split index varies fastest.
    const int split = (int)(blockIdx.x & (unsigned)(a.split_k - 1));
    const int tile = (int)(blockIdx.x >> a.split_shift);
    // (32-bit: the host guarantees split_k * ksteps < 2^31.)
    const int ka = (int)((unsigned)(split * a.ksteps) / (unsigned)a.split_k);
    const int kb = (int)((unsigned)((split + 1) * a.ksteps) / (unsigned)a.split_k);
    segment(tile, ka, kb, split, a.split_k);
  } else {
    // Stream-K: the ntiles * ksteps (tile, K-step) iterations, tile-major,
    // are dealt out in grid contiguous ranges, workgroup w taking
    // [w*I/grid, (w+1)*I/grid); the host guarantees grid <= I, so no range
    // is empty.  The workgroup holding iteration i is ((i+1)*grid - 1) / I,
    // which gives each tile's first contributor and contributor count.
    const unsigned long long I = (unsigned long long)a.ntiles * (unsigned)a.ksteps;
    const unsigned long long G = (unsigned)a.grid, w = blockIdx.x;
    const unsigned long long KS = (unsigned)a.ksteps;
    unsigned long long i0 = w * I / G;
    const unsigned long long i1 = (w + 1) * I / G;
    while (i0 < i1) {
      const unsigned long long t = i0 / KS;
      const int ka = (int)(i0 - t * KS);
      const unsigned long long kend = (unsigned long long)ka + (i1 - i0);
      const int kb = (int)(kend < KS ? kend : KS);
      const unsigned long long first = ((t * KS + 1) * G - 1) / I;
      const unsigned long long last = (((t + 1) * KS) * G - 1) / I;
      segment((int)t, ka, kb, (int)(w - first), (int)(last - first + 1));
      i0 += (unsigned long long)(kb - ka);
      if (i0 < i1) __syncthreads();  // LDS and is_last are reused by the next segment
    }
  }
}

template <int FMT, int MB, int NB, int WK, int WN, int U, int SWAP, int PACKED, int XL, int SK>
__global__ __launch_bounds__(64 * WK * WN) void gemm_kernel(GemmArgs a) {
  gemm_body<FMT, MB, NB, WK, WN, U, SWAP, PACKED, XL, SK, false>(a, nullptr, 0);
}

// An expert's entry count with its offsets clamped to the row list (so bad
// routing reads and writes nothing outside it).
__device__ __forceinline__ int moe_count(const MoeArgs& m, int e) {
  return min(m.offsets[e + 1], m.n_rows) - min(max(m.offsets[e], 0), m.n_rows);
}

// Compact grid: the slot-th expert, in expert order, with a positive count,
// or -1 if fewer experts have entries.  Every lane reads the offsets of
// four experts at once (E <= 256), so the search costs one round trip; the
// ballots make the result wave-uniform, and every wave of the workgroup
// computes the same value.
__device__ __forceinline__ int moe_active_expert(const MoeArgs& m, int slot) {
  const int lane = threadIdx.x & 63;
  bool act[kMoeCompactMaxE / 64];
#pragma unroll
  for (int i = 0; i < kMoeCompactMaxE / 64; ++i) {
    const int e = 64 * i + lane;
    act[i] = e < m.n_experts && moe_count(m, e) > 0;
  }
  int j = slot;
#pragma unroll
  for (int i = 0; i < kMoeCompactMaxE / 64; ++i) {
    const unsigned long long b = __ballot(act[i]);
    const int c = __popcll(b);
    if (j < c) {
      const unsigned long long below = b & ((1ull << lane) - 1ull);
      const unsigned long long hit = __ballot(act[i] && __popcll(below) == j);
      return 64 * i + __builtin_ctzll(hit);
    }
    j -= c;
  }
  return -1;
}

// MoE grouped GEMM: blockIdx.y is the expert (compact grid: the
// blockIdx.y-th expert with entries); its rows are entries [offsets[e],
// offsets[e+1]) of the routing (at most 16 * MB of them are computed), its
// weights, weight scales and shared-tile workspace are at the expert's
// strides, and its outputs are rows offsets[e].. of Y.
template <int FMT, int MB, int NB, int WK, int WN, int U, int SWAP, int PACKED, int XL, int SK>
__global__ __launch_bounds__(64 * WK * WN) void moe_gemm_kernel(GemmArgs a, MoeArgs m) {
  int e = blockIdx.y;
  if (m.compact) {
    e = moe_active_expert(m, e);
    if (e < 0) return;
  }
  const int off = min(max(m.offsets[e], 0), m.n_rows);
  const int rows = min(min(m.offsets[e + 1], m.n_rows) - off, 16 * MB);
  if (rows <= 0) return;  // an expert no token was routed to
  a.M = rows;
  a.wq += e * m.w_stride;
  a.sw += e * m.sw_stride;
  a.out = static_cast<char*>(a.out) + (long long)off * a.ldo * (a.out_mode ? 4 : 2);
  if (a.counters) {
    a.counters += (long long)e * a.ntiles * kCounterWords;
    a.part = static_cast<char*>(a.part) + e * m.part_stride;
  }
  gemm_body<FMT, MB, NB, WK, WN, U, SWAP, PACKED, XL, SK, true>(a, m.rows + off, m.xrow_max);
}

template <int FMT, int MB, int NB, int WK, int WN, int U, int SWAP, int PACKED, int XL, int SK>
hipError_t launch_gemm(const GemmArgs& a, dim3 grid, dim3 block, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<FMT, MB, NB, WK, WN, U, SWAP, PACKED, XL, SK>), grid, block, 0, s,
                     a);
  return hipGetLastError();
}

template <int FMT, int MB, int NB, int WK, int WN, int U, int SWAP, int PACKED, int XL, int SK>
hipError_t launch_moe_gemm(const GemmArgs& a, const MoeArgs& m, dim3 grid, dim3 block,
                           hipStream_t s) {
  hipLaunchKernelGGL((moe_gemm_kernel<FMT, MB, NB, WK, WN, U, SWAP, PACKED, XL, SK>), grid, block,
                     0, s, a, m);
  return hipGetLastError();
}

// Packs row-major codes [N, K] (row stride ldw) into the MFMA-native layout
// with T K-steps per MFMA (see the kernel header; T = 1 is the plain packed
// layout): one thread per 16-byte chunk, zero padding for rows >= N and bytes
// >= K.  Fragment f = (row block of R = 16/T rows, span of T K-steps) holds
// 16 x KSTEP bytes; its chunk (instruction jj, lane l) is the 16 bytes that
// lane l loads: row r = (l % 16) % R of the block, K-step t = (l % 16) / R of
// the span, bytes 64*jj + 16*(l / 16) of that K-step.
template <int KSTEP, int T>
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint8_t* __restrict__ w,
                                                          long long ldw, int N, int K,
                                                          int spans, uint8_t* __restrict__ out,
                                                          long long chunks) {
  constexpr int R = 16 / T;
  const long long c = blockIdx.x * 256LL + threadIdx.x;
  if (c >= chunks) return;
  constexpr int CHUNKS_PER_FRAG = 16 * KSTEP / 16;  // = KSTEP
  const long long f = c / CHUNKS_PER_FRAG;
  const int within = (int)(c % CHUNKS_PER_FRAG);
  const int jj = within / 64, l = within % 64;
  const long long nb = f / spans;
  const int sp = (int)(f % spans);
  const int p = l & 15;
  const long long row = nb * R + p % R;
  const long long k = (long long)(sp * T + p / R) * KSTEP + 64 * jj + 16 * (l >> 4);
  // (K % 16 == 0, so a chunk is either wholly inside K or wholly outside.)
  v4i v = {0, 0, 0, 0};
  if (row < N && k < K) v = *reinterpret_cast<const v4i*>(w + row * ldw + k);
  *reinterpret_cast<v4i*>(out + c * 16) = v;
}

}  // namespace w8
