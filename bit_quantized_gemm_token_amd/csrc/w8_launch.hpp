// Host-side declarations shared by the kernel translation units and the
// C-ABI: kernel argument blocks, launchers and the GEMM instance registry.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8 {

// ------------------------------------------------------------- quantizer --
struct QuantActArgs {
  const uint16_t* x;  // bf16 [M, K]
  uint8_t* xq;        // codes [M, K]
  float* sx;          // [M] or [M, K/128]
  long long ldx;      // elements
  long long ldq;      // bytes
  int M, K;
};

hipError_t launch_quantize_act(int fmt, const QuantActArgs& a, hipStream_t s);

struct QuantWeightArgs {
  const float* w;  // fp32 [N, K]
  uint8_t* wq;     // codes [N, K]
  float* sw;       // [N] or [ceil(N/128), ceil(K/128)]
  long long ldw;   // elements
  long long ldq;   // bytes
  int N, K;
};

hipError_t launch_quantize_weight(int fmt, const QuantWeightArgs& a, hipStream_t s);

// ------------------------------------------------------------------ GEMM --
struct GemmArgs {
  // Activation codes [M, K] (row stride ldq bytes), or for the fused
  // quantization (XL == 2) bf16 activations [M, K] (row stride ldq elements).
  const uint8_t* xq;
  const float* sx;         // activation scales (unused with XL == 2)
  const uint8_t* wq;       // weight codes [N, K], row stride ldw bytes
  const float* sw;         // weight scales
  void* out;               // bf16 Y [M, N] or 4-byte accumulators, stride ldo elements
  void* part;              // partials of shared tiles (workspace), 16-byte aligned
  unsigned int* counters;  // arrival counters, one per output tile
  long long ldq, ldw, ldo;
  int M, N, K;
  int ksteps;    // K-steps in total: ceil(K / KSTEP)
  int kfull;     // K-steps with no ragged tail: K / KSTEP
  int split_k;
  int split_shift;  // log2(split_k)
  int grid;      // 0: one workgroup per (tile, split); > 0: stream-K over this many
  int slots;     // partial slots per tile in the workspace
  int ntiles;    // output tiles along N (WN * NB row blocks each)
  int sgroups;   // Block_FP8: K / 128 (row stride of sx and sw)
  int out_mode;  // 0: bf16 Y; 1: raw accumulators
};

typedef hipError_t (*GemmLaunchFn)(const GemmArgs&, dim3 grid, dim3 block, hipStream_t);

struct GemmInstance {
  int fmt, mb, nb, wk, wn, unroll, swap, packed, xl;
  int sk;  // 1: the stream-K variant (cfg.grid > 0)
  GemmLaunchFn fn;
};

// MoE grouped GEMM: per-expert routing and strides (grid.y = experts).
struct MoeArgs {
  const int* offsets;      // [E + 1] routing offsets, ascending (device)
  const int* rows;         // [offsets[E]] activation row of each routed entry (device)
  long long w_stride;      // bytes between two experts' weights
  long long sw_stride;     // floats between two experts' weight scales
  long long part_stride;   // bytes between two experts' partials in the workspace
  int xrow_max;            // activation rows - 1 (row ids are clamped to [0, xrow_max])
  int n_rows;              // entries in `rows` (offsets are clamped to [0, n_rows])
  int n_experts;           // E
  int compact;             // 1: grid.y < E slots, slot j runs the j-th expert with entries
};

// Largest E for the compact grid (each lane of a wave reads the offsets of
// kMoeCompactMaxE / 64 experts at once).
constexpr int kMoeCompactMaxE = 256;

typedef hipError_t (*MoeLaunchFn)(const GemmArgs&, const MoeArgs&, dim3 grid, dim3 block,
                                  hipStream_t);

struct MoeInstance {
  int fmt, mb, nb, wk, wn, unroll, swap, packed, xl;
  int sk;  // 1: the stream-K variant (cfg.grid > 0)
  MoeLaunchFn fn;
};

// Weight layouts: 0 row-major; T in {1, 2, 4, 8} the packed layout with T
// K-steps per MFMA (1: blocks of 16 rows, the plain packed layout; 2, 4, 8:
// K-segmented, blocks of 16/T rows).
inline bool layout_valid(int layout) {
  return layout == 0 || layout == 1 || layout == 2 || layout == 4 || layout == 8;
}
inline int layout_segments(int layout) { return layout > 1 ? layout : 1; }
// Weight rows per block of the layout (row-major: the 16 of an MFMA).
inline int layout_rows(int layout) { return 16 / layout_segments(layout); }

// Packs row-major weight codes into packed layout `layout` (1, 2, 4 or 8).
hipError_t launch_pack_weight(int fmt, const uint8_t* w, long long ldw, int N, int K,
                              uint8_t* out, int layout, hipStream_t s);
// Spans (K-steps per MFMA of the layout) that cover K.
inline int layout_spans(int fmt, int K, int layout) {
  const int kstep = fmt == 1 ? 64 : 128;
  const int T = layout_segments(layout);
  return ((K + kstep - 1) / kstep + T - 1) / T;
}
inline size_t packed_weight_bytes(int fmt, int N, int K, int layout) {
  const int kstep = fmt == 1 ? 64 : 128;
  const int R = layout_rows(layout);
  return (size_t)((N + R - 1) / R) * layout_spans(fmt, K, layout) * 16 * kstep;
}

// Every compiled instance, gathered from the per-format translation units.
const GemmInstance* gemm_instances(int* count);
const MoeInstance* moe_instances(int* count);

// K-step (bytes of K per MFMA) of each format.
inline int kstep_of(int fmt) { return fmt == 1 ? 64 : 128; }

// Activations staged in LDS (cfg.x_lds): at most this many 1 KiB chunks (one
// per K-step, 16-row block of M and 64 bytes of K-step) per workgroup
// segment, 64 KiB, so two workgroups fit in a compute unit's 160 KiB.
constexpr int kXlChunks = 64;
// Fused quantization of Block_FP8 keeps each staged group's scales in LDS:
// at most this many K-steps per segment (kXlChunks / 2 chunks per K-step).
constexpr int kXlMaxGroups = kXlChunks / 2;

// Workspace layout: a fixed 2 MiB counter region (one 4-byte arrival counter
// per output tile in its own 128-byte cache line -- counters of neighbouring
// tiles sharing a line serialize their device-scope atomics -- for at most
// kSplitKMaxTiles tiles), then the partials: one 1 KiB fragment (64 lanes x
// 16 bytes) per (tile, slot, 16-row block of N, 16-row block of M), with
// split_k slots per tile for Split-K and stream_k_slots() for stream-K.  The
// counter region has the same size for every shape, so the partials of one
// call never overlap the counters of another call that shares the
// workspace, which keeps every counter at a multiple of 256 between calls
// (a Split-K launch adds exactly 256 to each of its tiles' counters; a
// stream-K launch counts in the line's second word and resets it).
constexpr int kSplitKMaxTiles = 16384;
constexpr int kCounterWords = 32;  // counter stride, 128 bytes
inline size_t ws_counter_bytes(int ntiles) {
  (void)ntiles;
  return (size_t)kSplitKMaxTiles * kCounterWords * 4;
}
inline size_t ws_partial_bytes(int ntiles, int slots, int row_blocks, int mb) {
  return (size_t)ntiles * slots * row_blocks * mb * 1024;
}
// Stream-K: an upper bound on the workgroups that share one tile of ks
// K-steps when I = ntiles * ks iterations are dealt to grid workgroups in
// ranges of at least floor(I / grid) >= 1: the first and last contributors
// hold at least one iteration each, every other one at least floor(I/grid).
inline int stream_k_slots(long long ntiles, int ks, int grid) {
  const long long I = ntiles * ks;
  const long long lmin = I / grid;
  if (ks <= 1) return 1;
  return (int)((ks - 2) / lmin) + 2;
}

}  // namespace w8
