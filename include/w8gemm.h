/*
 * w8gemm: small-M 8-bit quantized linear-layer GEMM for MI355X (gfx950).
 *
 *     Y[M, N] = dequant(Xq)[M, K] . dequant(Wq)[N, K]^T,   1 <= M <= 32
 *
 * The method: ai-radar.it, "Helion nel backend vLLM: un solo GEMM, tuning per
 * forma e guadagni fino al 10%".
 *   - paragraph 1: the three 8-bit formats FP8_Dynamic, W8A8_INT8, Block_FP8;
 *   - paragraph 2: Standard, Split-K and Swap-AB computed by one GEMM family;
 *   - paragraph 3: split_k and swap_ab are tunables, split_k a power of two
 *     up to 256, chosen per shape by an ahead-of-time tuner;
 *   - paragraph 4: the tuned kernels serve token counts up to 32 under graph
 *     replay; larger M goes to another backend;
 *   - paragraphs 6-7: per-shape config files, with a default config when no
 *     tuned entry exists;
 *   - paragraph 8: quantization is an auxiliary kernel beside the GEMM;
 *     w8_linear also offers it fused into the GEMM (one launch per layer).
 * The page defines none of the formats; this library uses:
 *   FP8_Dynamic  activations: per-token (row) OCP E4M3FN codes, fp32 sx[M];
 *                weights: E4M3FN codes, fp32 sw[N] (one per output channel);
 *                fp32 accumulation.
 *   W8A8_INT8    activations: per-token int8 codes, fp32 sx[M];
 *                weights: int8 codes, fp32 sw[N]; exact int32 accumulation
 *                (exact for any codes up to K = 133144, where K * 127^2
 *                reaches 2^31; beyond it, as far as the sums stay in int32).
 *   Block_FP8    activations: E4M3FN, fp32 sx[M, K/128] (1x128 groups);
 *                weights: E4M3FN, fp32 sw[ceil(N/128), K/128] (128x128
 *                blocks); each 128-wide K group's partial dot product is
 *                multiplied by sx[m, g] * sw[n/128, g] before the groups are
 *                summed in fp32.
 * Scales are dequantization multipliers (x ~= code * s).  Quantization uses
 * s = amax / Qmax (Qmax 448 for E4M3FN, 127 for int8; s = 1 for an all-zero
 * group), codes = round-to-nearest-even(x / s) with saturation to +-Qmax.
 * Output Y is bf16 (round to nearest even), row-major.
 *
 * Layouts: every matrix is row-major with an explicit leading dimension.
 * Wq is [N, K] with K contiguous (the usual linear-layer weight layout).
 *
 * Ownership: the caller owns every device buffer.  w8_quantize_act,
 * w8_gemm_w8a8 and w8_gemm_w8a8_acc never allocate, free or synchronize; they
 * only enqueue kernels on the caller's stream, so they can be captured into a
 * HIP graph.  The config table is owned by the library (process-global,
 * guarded by a mutex).  The tuners (w8_tune_shape, w8_moe_tune,
 * w8_profile_configs) allocate and synchronize: they return W8_E_INVALID,
 * having done nothing, when opts->stream or the null stream is capturing.
 *
 * Errors: every entry point returns a w8_status.  All argument checks run
 * before anything is enqueued, and nothing throws or aborts across the ABI.
 * A kernel launch failure returns W8_E_HIP; asynchronous device faults show
 * up at the caller's next synchronization.  w8_last_error() gives a
 * thread-local message for the last failing call.
 *
 * Streams: w8_stream is a hipStream_t passed as a plain pointer (NULL is the
 * default stream).  Device pointers are HIP device (or managed) addresses.
 */
#ifndef W8GEMM_H
#define W8GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W8_ABI_VERSION 5
#define W8_MAX_M 32         /* token-count window of the tuned path (paragraph 4) */
#define W8_MAX_SPLIT_K 256  /* split_k is a power of two up to 256 (paragraph 3) */
#define W8_GROUP 128        /* Block_FP8 group / block edge */

typedef void *w8_stream; /* hipStream_t */

/* The operations configs are tuned for: the GEMM on quantized activations
 * (w8_gemm_w8a8), the whole linear layer (w8_linear), and the MoE grouped
 * GEMM on quantized activations (w8_moe_gemm) and on bf16 activations with
 * the quantization fused (w8_moe_linear).  The two MoE ops' table entries
 * hold the token count T in the M field and take w8_moe_tune, not
 * w8_tune_shape.                                                           */
typedef enum {
    W8_OP_GEMM = 0,
    W8_OP_LINEAR = 1,
    W8_OP_MOE = 2,
    W8_OP_MOE_LINEAR = 3
} w8_op;

typedef enum {
    W8_FP8_DYNAMIC = 0,
    W8_W8A8_INT8 = 1,
    W8_BLOCK_FP8 = 2
} w8_fmt;

typedef enum {
    W8_OK = 0,
    W8_E_INVALID = 1,      /* bad argument, alignment or config */
    W8_E_UNSUPPORTED = 2,  /* outside the method's window (M > 32): caller falls back */
    W8_E_WORKSPACE = 3,    /* workspace missing or too small */
    W8_E_TABLE_FORMAT = 4, /* config-table file malformed; the old table is kept */
    W8_E_IO = 5,           /* file could not be read or written */
    W8_E_HIP = 6,          /* a HIP runtime call failed */
    W8_E_VALIDATION = 7,   /* tuner: no candidate passed validation */
    W8_E_NOT_FOUND = 8     /* lookup miss */
} w8_status;

/* One kernel configuration of the GEMM family (paragraphs 2-3 of the page:
 * the algorithmic variants are parameters, not separate kernels).
 *   tile_n   output columns (= weight rows) each wave owns: 16, 32 or 64
 *            (one activation fragment feeds tile_n/16 MFMAs per K-step);
 *            on the K-segmented layouts (below) 1, 2 or 4 blocks of the
 *            layout's 16/T rows: T = 2: 8, 16, 32; T = 4: 4, 8, 16;
 *            T = 8: 2, 4, 8.
 *   waves_k  wavefronts of a workgroup that split its K range and are
 *            reduced through LDS: 1, 2, 4, 8 or 16.
 *   waves_n  wavefronts of a workgroup side by side along N, which share
 *            the activations staged in LDS: 1, 2, 4 or 8; a workgroup covers
 *            tile_n * waves_n columns.  waves_n > 1 needs waves_k == 1 and
 *            x_lds == 1.
 *   x_lds    0: each wave loads its activation fragments from memory inside
 *            the K loop.  1: the workgroup first copies the activations of
 *            its K range into LDS and the K loop reads them there; needs
 *            waves_k <= 8 and at most 64 KiB per workgroup:
 *            ceil(M/16) x (K-steps per workgroup) x (K-step bytes / 64) <= 64,
 *            with K-steps per workgroup = ceil(K-steps / split_k), or for
 *            stream-K min(K-steps, ceil(tiles x K-steps / grid)).
 *   unroll   K-steps each wave loads per stage (two stages in flight):
 *            1, 2 or 4, with tile_n/16 * unroll <= 4.
 *   split_k  workgroups splitting K, reduced in fixed order by the last one
 *            to finish: 1, 2, 4, ..., 256 (Split-K; 1 = Standard).
 *   grid     0: one workgroup per (output tile, split).  > 0: stream-K, a
 *            decomposition for a GPU with many compute units and few tiles:
 *            exactly `grid` workgroups share the (tile, K-step) iterations
 *            in equal contiguous ranges; a tile split between workgroups is
 *            reduced like a split-K tile.  Needs split_k == 1 and grid at
 *            most tiles x K-steps.
 *   swap_ab  0: MFMA A operand = activations, B = weights^T.
 *            1: Swap-AB, Y^T = Wq . Xq^T: A = weights, B = activations^T.
 *   quant_launch  W8_OP_LINEAR and W8_OP_MOE_LINEAR only (0 for the other
 *            ops).  0: the activations are quantized inside the GEMM: staged
 *            in LDS (x_lds == 1, waves_k <= 4), or for the Block_FP8 linear
 *            op also in the K loop (x_lds == 0, tile_n 16 or 32, waves_n 1,
 *            waves_k 2, 4 or 8, unroll 1).  1: they are quantized by a
 *            launch of their own
 *            (w8_quantize_act's kernel) into the workspace, and the GEMM
 *            runs with this config under the W8_OP_GEMM rules.  The tuner
 *            tries both for the linear op and keeps the faster.
 * Set abi_version to W8_ABI_VERSION and reserved[] to 0.  The weight layout
 * (row-major, packed or K-segmented packed, below) is a property of the
 * weight buffer, not of the config: it is given by the ldw argument of the
 * GEMM.  On the K-segmented layouts a config has x_lds 0, waves_n 1, grid 0
 * and, for the linear op, quant_launch 1.                                  */
typedef struct {
    int32_t abi_version;
    int32_t tile_n;
    int32_t waves_k;
    int32_t waves_n;
    int32_t unroll;
    int32_t split_k;
    int32_t grid;
    int32_t swap_ab;
    int32_t x_lds;
    int32_t quant_launch;
    int32_t reserved[1];
} w8_cfg;

/* Options of the ahead-of-time tuner (paragraph 3 and 6 of the page). */
typedef struct {
    int32_t abi_version;      /* W8_ABI_VERSION */
    int32_t warmup;           /* untimed graph replays per candidate (default 2) */
    int32_t replays;          /* timed graph replays per candidate and bank (default 5) */
    int32_t bank2_top;        /* best bank-1 candidates re-timed on bank 2 (default 5) */
    int64_t rotate_bytes;     /* weight bytes cycled through per graph, >= the last-level
                                 cache so reads come from HBM (default 512 MiB) */
    int32_t max_split_k;      /* largest split_k tried (default 256) */
    int32_t insert;           /* 1: insert the winner into the config table */
    int32_t fail_candidate;   /* test hook: candidate with this index fails validation
                                 (-1 = none) */
    int32_t packed;           /* weight layout tuned: 0 row-major, 1 packed, 2/4/8
                                 K-segmented packed (the grouped GEMM: 0 or 1) */
    int32_t stream_k;         /* 1: also try stream-K grids (default 0: on the
                                 shapes measured so far they never won) */
    int32_t op;               /* w8_op tuned (default W8_OP_GEMM) */
    int32_t top_n;            /* > 0: time only the top_n candidates of the cost
                                 model's ranking (w8_rank_configs); 0: all */
    w8_stream stream;         /* the caller's stream: the tuners allocate and
                                 synchronize, so they refuse to run (W8_E_INVALID,
                                 nothing done) while this stream or the null stream
                                 is being captured into a graph (default NULL: the
                                 null stream only) */
} w8_tune_opts;

typedef struct {
    int32_t candidates;       /* feasible candidates enumerated */
    int32_t validated;        /* of which passed validation against the default config */
    int32_t rejected;         /* of which failed validation */
    int32_t best_index;       /* index of the winner in enumeration order; -1: the
                                 default config, not a candidate, won on bank 2 */
    double best_us_bank1;     /* winner, median us per GEMM on timing bank 1 */
    double best_us_bank2;     /* winner, median us per GEMM on bank 2 (reported figure) */
    double default_us_bank2;  /* default config on bank 2 (it competes there: the
                                 winner is never slower; 0 if it failed validation) */
    double best_gbps;         /* algorithmic bytes / best_us_bank2 */
    double tune_seconds;      /* wall-clock time of the whole tuning call */
    double best_us_bank2_min; /* winner on bank 2: fastest replay, us per GEMM */
    double best_us_bank2_p90; /* winner on bank 2: 90th-percentile replay */
} w8_tune_stats;

/* ---------------------------------------------------------------- info -- */
int w8_abi_version(void);
const char *w8_status_string(w8_status s);
const char *w8_last_error(void); /* thread-local; "" when the last call succeeded */

/* --------------------------------------------------------- quantization -- */
/* Dynamic activation quantization (paragraph 1's formats, paragraph 8's
 * auxiliary quantization kernel).  One kernel launch on `stream`.
 *   x    bf16 [M, K], row stride ldx elements (device)
 *   xq   1-byte codes [M, K], row stride ldq bytes (device): E4M3FN for the
 *        FP8 formats, int8 for W8A8_INT8
 *   sx   fp32 scales (device): [M] (FP8_Dynamic, W8A8_INT8) or [M, K/128]
 *        row-major (Block_FP8)
 * Requires 1 <= M <= 32 (else W8_E_UNSUPPORTED), K >= 16, K % 16 == 0
 * (Block_FP8: K % 128 == 0), ldx >= K, ldq >= K, x 16-byte aligned with
 * ldx % 8 == 0, xq 16-byte aligned with ldq % 16 == 0.  Inputs must be finite. */
w8_status w8_quantize_act(w8_fmt fmt, int M, int K, const void *x, int64_t ldx,
                          void *xq, int64_t ldq, float *sx, w8_stream stream);

/* Offline weight quantization to E4M3FN (FP8_Dynamic: one scale per row,
 * sw[N]; Block_FP8: one scale per 128x128 block, sw[ceil(N/128), ceil(K/128)]
 * row-major, edge blocks may be partial).  W8A8_INT8 weights are supplied as
 * codes and scales and are rejected here (W8_E_INVALID).
 *   w    fp32 [N, K], row stride ldw elements (device)
 *   wq   1-byte codes [N, K], row stride ldq bytes (device)
 * Requires N >= 1, K >= 1, ldw >= K, ldq >= K.  Inputs must be finite.       */
w8_status w8_quantize_weight(w8_fmt fmt, int N, int K, const float *w, int64_t ldw,
                             void *wq, int64_t ldq, float *sw, w8_stream stream);

/* ------------------------------------------------------------------ GEMM -- */
/* Weight layouts (the "memory layout" choice the page puts in the tuner's
 * search space, paragraph 3), each with a code used by the config, table
 * and tuner functions:
 *   0  row-major: codes [N, K], row stride ldw bytes (ldw >= K,
 *      ldw % 16 == 0).
 *   1  packed: the MFMA-native layout written by w8_pack_weight: for each
 *      block of 16 rows and each K-step (64 bytes of K for W8A8_INT8, 128
 *      for the FP8 formats), the 16 x K-step bytes are stored in the order
 *      the kernel's lanes load them, so every load instruction reads 1 KiB
 *      contiguous; rows and K are zero-padded to whole fragments.  GEMM
 *      calls pass ldw = 0.
 *   T = 2, 4, 8  K-segmented packed: one MFMA takes 16/T weight rows times
 *      T consecutive K-steps (and 16/T tokens times the same K-steps); of
 *      its products only the T diagonal blocks are kept and summed.  The
 *      fragments (16/T rows, T K-steps) are stored like layout 1's, rows
 *      zero-padded to multiples of 16/T and K to multiples of T K-steps.  At
 *      M <= 16/T tokens the same weight bytes make T times as many output
 *      tiles, which fills the GPU on narrow N without splitting K.  Larger M
 *      runs as consecutive launches of 2 x 16/T tokens.  GEMM calls pass
 *      ldw = -T.
 * Configs are tuned per layout.                                            */

/* Bytes of packed layout `layout` (1, 2, 4 or 8) for an N x K weight of fmt. */
w8_status w8_packed_weight_size(w8_fmt fmt, int N, int K, int layout, size_t *bytes);

/* Packs row-major codes (device, 16-byte aligned, ldw >= K, ldw % 16 == 0)
 * into wp (device, 16-byte aligned, w8_packed_weight_size bytes) in layout
 * 1, 2, 4 or 8.  Offline; one kernel launch on stream.  Same preconditions
 * on N and K as the GEMM. */
w8_status w8_pack_weight(w8_fmt fmt, int N, int K, const void *wq, int64_t ldw, void *wp,
                         int layout, w8_stream stream);

/* Bytes of device workspace operation op needs for (fmt, M, N, K) under cfg
 * on weights of layout `packed` (0, 1, 2, 4 or 8; cfg NULL: the config
 * w8_resolve_config picks for op and that layout).  The GEMM needs none when no tile
 * is shared between workgroups (split_k == 1 and grid == 0); otherwise a
 * fixed 2 MiB region of arrival counters, then the partials of shared
 * tiles, so split_k > 1 and grid > 0 support at most 16384 output tiles
 * (N <= 16384 * tile_n * waves_n).  The linear op with quant_launch == 1
 * adds, after the GEMM's part and never below the 2 MiB counter region (so a
 * workspace shared by any sequence of calls keeps its counters intact),
 * the codes (M rows of K rounded up to 16 bytes) and the scales of the
 * activations, each region 256-byte aligned.                               */
w8_status w8_workspace_size(w8_fmt fmt, w8_op op, int M, int N, int K, int packed,
                            const w8_cfg *cfg, size_t *bytes);

/* The quantized GEMM.  One kernel launch on `stream` (the split-K reduction
 * runs inside it: the last workgroup of each output tile to finish sums the
 * partials in split order, so results are run-to-run deterministic).
 *   xq, sx  activations as written by w8_quantize_act
 *   wq, sw  weights: codes in the row-major layout (row stride ldw bytes),
 *           with ldw = 0 in the packed layout, with ldw = -2, -4 or -8 in
 *           that K-segmented layout; scales in the layout given above for fmt
 *   y       bf16 [M, N], row stride ldy elements (device)
 *   cfg     kernel configuration; NULL = w8_resolve_config's pick for
 *           (fmt, weight layout, M, N, K): table entry, M-bucket entry or
 *           the cost model's pick
 *   ws      workspace of at least w8_workspace_size() bytes, zero-filled
 *           before its first use; every completed call leaves its arrival
 *           counters at multiples of 256 (split-K adds 256 to each of its
 *           tiles' counters per call, stream-K returns its own to zero), the
 *           state the next call needs, so it is never cleared again.  May be
 *           NULL when the size is 0.  Calls that share
 *           a workspace must not run concurrently.
 * Requires 1 <= M <= 32 (else W8_E_UNSUPPORTED), N >= 1, K >= 16,
 * K % 16 == 0 (Block_FP8: K % 128 == 0), ldq >= K, ldy >= N, xq/wq 16-byte
 * aligned with ldq % 16 == 0, finite codes (no E4M3FN NaN codes).          */
w8_status w8_gemm_w8a8(w8_fmt fmt, int M, int N, int K,
                       const void *xq, int64_t ldq, const float *sx,
                       const void *wq, int64_t ldw, const float *sw,
                       void *y, int64_t ldy, const w8_cfg *cfg,
                       void *ws, size_t ws_bytes, w8_stream stream);

/* Test hook: the same GEMM with the accumulators written raw instead of the
 * bf16 output.  acc is [M, N] 4-byte elements with row stride ldacc:
 *   W8A8_INT8    int32  sum_k xq*wq               (exact)
 *   FP8_Dynamic  fp32   sum_k dec(xq)*dec(wq)     (scales not applied)
 *   Block_FP8    fp32   sum_g sx*sw*partial_g     (the value before bf16)  */
w8_status w8_gemm_w8a8_acc(w8_fmt fmt, int M, int N, int K,
                           const void *xq, int64_t ldq, const float *sx,
                           const void *wq, int64_t ldw, const float *sw,
                           void *acc, int64_t ldacc, const w8_cfg *cfg,
                           void *ws, size_t ws_bytes, w8_stream stream);

/* w8_gemm_w8a8 for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without a workspace, the same kernels and results.  A config
 * that shares output tiles (split_k > 1 or grid > 0) keeps its arrival
 * counters and partials in a 16 MiB device array of the library's own (2
 * MiB of counters, then up to 14 MiB of partials), which each GPU the
 * library runs on holds until the process ends; a config that needs more
 * returns W8_E_WORKSPACE before anything is launched.  It allocates
 * nothing, frees nothing and never synchronizes.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on several
 * streams) race and must not be made. */
w8_status w8_gemm_w8a8_noalloc(w8_fmt fmt, int M, int N, int K,
                               const void *xq, int64_t ldq, const float *sx,
                               const void *wq, int64_t ldw, const float *sw,
                               void *y, int64_t ldy, const w8_cfg *cfg, w8_stream stream);

/* The whole linear layer on bf16 activations.  With quant_launch == 0, one
 * kernel launch: activation quantization (the w8_quantize_act rules, giving
 * the same codes and scales) fused into the GEMM.  With x_lds == 1 each
 * workgroup quantizes the activations of its K range into LDS: per 1x128
 * group for Block_FP8; per token for the other formats, after a pass over
 * the whole row for its absolute maximum.  With x_lds == 0 (Block_FP8 only)
 * each wave quantizes the 1x128 groups it loads inside the K loop.  Either
 * way Y equals w8_quantize_act followed by w8_gemm_w8a8 with the same tile
 * config, bit for bit.
 *   x       bf16 [M, K], row stride ldx elements (device), 16-byte aligned,
 *           ldx % 8 == 0
 *   wq, sw, y, ws, stream  as for w8_gemm_w8a8
 *   cfg     NULL = w8_resolve_config's pick for (fmt, W8_OP_LINEAR, weight
 *           layout, M, N, K).  With quant_launch == 1 the call makes two
 *           launches instead: w8_quantize_act's kernel into the workspace,
 *           then the GEMM (same Y).  Both forms allocate nothing.          */
w8_status w8_linear(w8_fmt fmt, int M, int N, int K, const void *x, int64_t ldx,
                    const void *wq, int64_t ldw, const float *sw,
                    void *y, int64_t ldy, const w8_cfg *cfg,
                    void *ws, size_t ws_bytes, w8_stream stream);

/* ---------------------------------------------------------------- config -- */
/* W8_OK if cfg is a valid configuration of operation op (GEMM or LINEAR;
 * grouped configs take w8_moe_validate_config) for (fmt, M, N, K) on
 * weights of layout `layout` (0, 1, 2, 4 or 8), else
 * W8_E_INVALID (with the reason in w8_last_error()).                        */
w8_status w8_validate_config(w8_fmt fmt, w8_op op, int M, int N, int K, int layout,
                             const w8_cfg *cfg);

/* The built-in rule-of-thumb configuration of op for (fmt, M, N, K): fixed
 * tile and waves, Swap-AB below 32 tokens, the smallest split_k that fills
 * the machine (paragraph 7 of the page: a default config serves untuned
 * shapes); on the K-segmented layouts one block per wave and two K-waves.
 * The tuner validates every candidate against its output.                 */
w8_status w8_default_config(w8_fmt fmt, w8_op op, int M, int N, int K, int layout,
                            w8_cfg *out);

/* The cost model's pick (the top-1 of w8_rank_configs with the default
 * options for op and layout): what an untuned shape runs
 * (flashinfer-ai/flashinfer pull 3948: a heuristic top-1 without tuning). */
w8_status w8_model_config(w8_fmt fmt, w8_op op, int M, int N, int K, int packed, w8_cfg *out);

/* The cost model's predicted microseconds per call, us[i], of config
 * cfgs[i] for operation op[i] (W8_OP_GEMM or W8_OP_LINEAR) on
 * (fmt[i], M[i], N[i], K[i]) with weights of layout layout[i], for i < n.
 * params NULL: the compiled constants; else nparams = 13 constants in the
 * order t0, cu_bw, latency, hbm_bw, slots, sk_base, sk_slot, xl_stage,
 * wg_cost, mfma, reduce, q_launch, q_row_bw (the model's fitter passes its
 * trial values here, so fit and library evaluate the same model).  Host
 * only; the configs are not validated beyond what the arithmetic needs
 * (positive shape and config fields, a known layout: else W8_E_INVALID). */
w8_status w8_predict_us(int n, const int *fmt, const int *op, const int *layout,
                        const int *M, const int *N, const int *K, const w8_cfg *cfgs,
                        const double *params, int nparams, double *us);

/* The config op uses when called with cfg == NULL for weights in the given
 * layout (packed = 0 row-major, 1 packed, 2/4/8 K-segmented), looked up for
 * this device's arch
 * and W8_ABI_VERSION: the table entry for (fmt, op, layout, M, N, K)
 * (*from_table = 1); else the entry for the same (fmt, op, layout, N, K)
 * whose M is nearest in the same floor(log2 M) bucket (the larger on a tie)
 * and whose config is valid for M (*from_table = 2); else the cost model's
 * pick, w8_model_config (*from_table = 0).                                 */
w8_status w8_resolve_config(w8_fmt fmt, w8_op op, int M, int N, int K, int packed,
                            w8_cfg *out, int *from_table);

/* ----------------------------------------------------------- config table -- */
/* Per-shape config table (paragraphs 6-7 of the page).  Text format, one entry
 * per line:
 *   arch abi fmt op layout M N K tile_n waves_k waves_n unroll split_k grid
 *   swap_ab x_lds quant_launch us_per_call
 * with op "gemm", "linear", "moe" or "moe_linear" and layout "row",
 * "packed", "seg2", "seg4" or "seg8" (codes 0, 1, 2, 4, 8); '#' starts a
 * comment.  Entries whose arch or
 * abi differ from this build and device are kept in the file but never used.
 * w8_load_config_table replaces the in-memory table atomically: on any parse
 * error it returns W8_E_TABLE_FORMAT (line number in w8_last_error()) and
 * keeps the old table.  If the environment variable W8_CONFIG_TABLE names a
 * file, it is loaded at the first config lookup.                           */
w8_status w8_load_config_table(const char *path);
w8_status w8_save_config_table(const char *path);
void w8_clear_config_table(void);
int w8_config_table_size(void);
/* Entries of the last load that were skipped for a foreign arch or abi. */
int w8_config_table_foreign(void);
/* Insert or replace one entry for this device (validated first; a MOE
 * entry against the GEMM rules at M = T, and again against the grouped
 * kernel's rules when w8_moe_config reads it). */
w8_status w8_set_config(w8_fmt fmt, w8_op op, int M, int N, int K, int packed,
                        const w8_cfg *cfg, double us_per_call);
/* Exact lookup for this device: W8_OK on a hit (with the entry's time per
 * call in *us_per_call when not NULL), W8_E_NOT_FOUND on a miss.  Comparing
 * the two layouts' times tells a caller which layout to store its weights in. */
w8_status w8_lookup_config(w8_fmt fmt, w8_op op, int M, int N, int K, int packed,
                           w8_cfg *out, double *us_per_call);

/* ------------------------------------------------------------------ tuner -- */
/* Ahead-of-time per-shape tuner (paragraph 3 of the page: the autotuner
 * compares configurations and keeps the best for each shape).  Tunes one
 * operation (opts->op) for one weight layout (opts->packed).  Allocates its
 * own inputs (random codes, bf16 activations for W8_OP_LINEAR, and scales),
 * enumerates the configs of the family (W8_OP_LINEAR: the fused ones, with
 * x_lds and waves_k <= 4, plus quant_launch = 1 with the GEMM's config for
 * the shape and layout -- table entry or model pick -- and with the GEMM's
 * default, so tune the GEMM first)
 * (tile_n x (waves_k or waves_n) x x_lds x unroll x (split_k in {1, 2, ...,
 * max_split_k}, or with opts->stream_k a stream-K grid in {256, 512, 1024})
 * x swap_ab) minus those that cannot pay off or duplicate another (fewer
 * than one K-step per wave, unroll above the K-steps per wave, partials
 * above twice the weight bytes, fewer than min(256, most possible) waves);
 * with opts->top_n > 0 only the top_n of the cost model's ranking remain
 * (w8_rank_configs).  It checks each
 * against the default GEMM config's output (for W8_OP_LINEAR after the
 * standalone quantizer; bit-equal for W8A8_INT8, within 1e-2 relative for
 * the FP8 formats) and times it as HIP graph replays over
 * rotating weight copies; the best on timing bank 1 are re-timed on bank 2,
 * together with the op's default config (validated like a candidate), and
 * the bank-2 winner is returned (and inserted into the table when
 * opts->insert): the default unless a candidate is strictly faster, so the
 * entry is never slower than the default on bank 2.  opts NULL = defaults.
 * Synchronizes the device; W8_E_INVALID (nothing done) while opts->stream or
 * the null stream is capturing.                                            */
w8_status w8_tune_shape(w8_fmt fmt, int M, int N, int K, const w8_tune_opts *opts,
                        w8_cfg *best, w8_tune_stats *stats);
void w8_tune_default_opts(w8_tune_opts *opts);

/* The tuner's candidate set for (fmt, M, N, K) under opts (op, packed,
 * max_split_k, stream_k; top_n is ignored), ranked by the cost model's
 * predicted us per call, ascending.  The model (flashinfer-ai/flashinfer
 * pull 3948: score every feasible tactic, profile only the top-N) charges a
 * fixed launch cost, the busiest compute unit's vector-memory bytes at a
 * Little's-law rate (bytes in flight over load latency, capped), the HBM
 * time of the weights (overlapped), and the reduction chain, LDS staging and
 * quantization costs, with constants fitted to measured timings.  Writes up
 * to cap configs (and their predictions when predicted_us is not NULL) and
 * the set's size in *count.  Host only: no device call.                    */
w8_status w8_rank_configs(w8_fmt fmt, int M, int N, int K, const w8_tune_opts *opts,
                          w8_cfg *out, double *predicted_us, int cap, int *count);

/* Times n configs of opts->op with the tuner's harness (same inputs,
 * validation against the default GEMM config, median us per call of graph
 * replays over rotating weight copies; bank 1 only, nothing inserted):
 * valid[i] = 1 and us[i] the time, or valid[i] = 0 and us[i] = 0 for a
 * config whose output failed validation.  Allocates and synchronizes, like
 * w8_tune_shape.                                                           */
w8_status w8_profile_configs(w8_fmt fmt, int M, int N, int K, const w8_tune_opts *opts,
                             const w8_cfg *cfgs, int n, double *us, int *valid);

/* --------------------------------------------------------------- MoE -- */
/* MoE grouped GEMM in the same three formats (paragraph 9 of the page: MoE
 * models, where the MoE backend becomes the main optimization target, are
 * the next stated goal).  E experts share (N, K).  T token rows were
 * quantized once (w8_quantize_act: xq [T, K], sx [T] or [T, K/128]); the
 * routing lists, per expert e, the routed entries i in [offsets[e],
 * offsets[e+1]) and the token row rows[i] of each, and entry i's output is
 *   Y[i, :] = dequant(xq[rows[i]]) . dequant(Wq_e)^T
 * with expert e's weight codes Wq_e and scales sw_e in the format's
 * layout -- the GEMM of w8_gemm_w8a8 on the gathered rows, per expert.  One
 * kernel launch covers all experts (no host synchronization: the routing is
 * read on the device); an expert with no entry reads no weights.  When
 * 0 < n_rows < E <= 256 the launch holds n_rows expert slots instead of E
 * (ascending offsets leave at most n_rows experts with entries), slot j
 * running the j-th expert that has entries.
 *   offsets  int32 [E + 1] (device), ascending, offsets[0] = 0,
 *            offsets[E] = n_rows; each expert's count offsets[e+1] -
 *            offsets[e] must be <= max_m (rows past 16 ceil(max_m/16) of an
 *            expert are not computed).  Offsets are clamped to [0, n_rows],
 *            so bad routing never reads or writes outside rows and y (it
 *            may leave entries unwritten).
 *   rows     int32 [n_rows] (device), each in [0, T) (clamped if not);
 *            n_rows = 0: nothing is computed or launched (rows, y and ws
 *            may be NULL)
 *   max_m    bound on any expert's count, 1..32 (else W8_E_UNSUPPORTED);
 *            kernels for ceil(max_m / 16) row blocks run
 *   wq       expert e's codes at wq + e * w_stride bytes: row-major [N, K]
 *            with row stride ldw, or with ldw = 0 the packed layout
 *            (w8_pack_weight per expert); w_stride % 16 == 0
 *   sw       expert e's scales at sw + e * sw_stride floats
 *   y        bf16 [n_rows, N], row stride ldy (device), entry i's row i
 *   cfg      a GEMM-family config valid at M = max_m whose (waves_k, waves_n,
 *            x_lds) is one of (1|2|4|8, 1, 0) or (1, 2|4|8, 1); NULL =
 *            w8_moe_config's.  Shared tiles (split_k > 1 or grid > 0) need
 *            E x tiles <= 16384.
 *   ws       w8_moe_workspace_size bytes: the 2 MiB counter region, then
 *            each expert's partials; zero-filled before first use.
 * Same allocation, ordering and error rules as w8_gemm_w8a8.               */
w8_status w8_moe_gemm(w8_fmt fmt, int E, int T, int N, int K, int max_m,
                      const void *xq, int64_t ldq, const float *sx,
                      const int32_t *offsets, const int32_t *rows, int n_rows,
                      const void *wq, int64_t ldw, int64_t w_stride,
                      const float *sw, int64_t sw_stride, void *y, int64_t ldy,
                      const w8_cfg *cfg, void *ws, size_t ws_bytes, w8_stream stream);
/* Workspace bytes of w8_moe_gemm or w8_moe_linear with cfg (a config of
 * either; NULL = w8_moe_config's): the shared-tile region, and with
 * quant_launch the T tokens' codes and scales after it.                    */
w8_status w8_moe_workspace_size(w8_fmt fmt, int E, int T, int N, int K, int max_m, int packed,
                                const w8_cfg *cfg, size_t *bytes);
/* W8_OK if cfg is valid for w8_moe_gemm with these sizes and layout.       */
w8_status w8_moe_validate_config(w8_fmt fmt, int E, int N, int K, int max_m, int packed,
                                 const w8_cfg *cfg);
/* The config w8_moe_gemm uses for cfg == NULL: the table entry for
 * (fmt, W8_OP_MOE, layout, T, N, K) if it is valid for E and max_m; else
 * tile_n 32, one K-wave (two, with unroll 2, for T <= 2), no split, no
 * x_lds -- the fastest on 128-expert top-8 layers measured at 1..32
 * tokens -- or, where that is invalid, the cost model's fastest valid config
 * for a GEMM of N x min(E, 8 T) columns (the experts T tokens reach with up
 * to 8 each).  *from_table (may be NULL) is 1 for a table entry.           */
w8_status w8_moe_config(w8_fmt fmt, int E, int T, int N, int K, int max_m, int packed,
                        w8_cfg *out, int *from_table);

/* The MoE grouped GEMM on bf16 activations x [T, K] (row stride ldx,
 * 16-byte aligned, ldx % 8 == 0): the whole MoE expert layer from the
 * tokens.  With cfg->quant_launch == 0 the activation quantization is fused
 * into the grouped kernel: each expert's workgroups quantize the token rows
 * routed to it while their weights load, per token (FP8_Dynamic,
 * W8A8_INT8: the row's maximum over the whole of K) or per 1x128 group
 * (Block_FP8), with the codes and scales of w8_quantize_act; the config
 * needs x_lds == 1 and (waves_k, waves_n) in {(1, 4), (1, 8)}.
 * With quant_launch == 1 the tokens are quantized by a launch of their own
 * into the workspace (after its shared-tile region), then the grouped
 * kernel runs with the config under w8_moe_gemm's rules.  Either way Y
 * equals w8_quantize_act followed by w8_moe_gemm with the same tiling, bit
 * for bit.  NULL cfg = w8_moe_linear_config.  All other arguments, rules
 * and the workspace (w8_moe_workspace_size with the resolved cfg) as for
 * w8_moe_gemm.                                                           */
w8_status w8_moe_linear(w8_fmt fmt, int E, int T, int N, int K, int max_m,
                        const void *x, int64_t ldx,
                        const int32_t *offsets, const int32_t *rows, int n_rows,
                        const void *wq, int64_t ldw, int64_t w_stride,
                        const float *sw, int64_t sw_stride, void *y, int64_t ldy,
                        const w8_cfg *cfg, void *ws, size_t ws_bytes, w8_stream stream);
/* The config w8_moe_linear uses for cfg == NULL: the table entry for
 * (fmt, W8_OP_MOE_LINEAR, layout, T, N, K) if it is valid for E and max_m;
 * else w8_moe_config's config with quant_launch = 1.  *from_table (may be
 * NULL) is 1 for a table entry.                                           */
w8_status w8_moe_linear_config(w8_fmt fmt, int E, int T, int N, int K, int max_m, int packed,
                               w8_cfg *out, int *from_table);

/* Ahead-of-time tuning of the MoE grouped GEMM for E experts of (N, K) at T
 * tokens routed top-k (1 <= topk <= E): the grouped GEMM's configs
 * (w8_moe_validate_config with max_m = T), each checked against the default
 * config's output and timed like w8_tune_shape's candidates, as graphs of
 * calls over rotating weight copies and seeded uniform top-k routings (up
 * to 64 calls, each with its own routing, so that the experts one graph
 * reaches span opts->rotate_bytes);
 * opts as for w8_tune_shape (stream_k and top_n ignored); opts->op =
 * W8_OP_GEMM tunes w8_moe_gemm, W8_OP_LINEAR tunes w8_moe_linear (fused
 * quantization, checked against w8_quantize_act + the fallback config).
 * The winner is inserted as the (fmt, W8_OP_MOE or W8_OP_MOE_LINEAR,
 * layout, T, N, K) entry when opts->insert.  Allocates and synchronizes.  */
w8_status w8_moe_tune(w8_fmt fmt, int E, int T, int N, int K, int topk,
                      const w8_tune_opts *opts, w8_cfg *best, w8_tune_stats *stats);

/* -------------------------------------------------------- measurement -- */
/* The read floor the GEMM is measured against: one kernel launch on `stream`
 * that reads `bytes` of device memory from `src` once (16-byte non-temporal
 * loads, 1 KiB per wave instruction, the chunks dealt to the grid's waves
 * interleaved, `depth` chunks per wave in flight) and writes one word per
 * wave to `sink`.  A GEMM that streams the same bytes in one launch cannot
 * take less time; the benchmark graph-replays it over the same rotating
 * weight buffers as the GEMM and reports each GEMM's time against the best
 * of a few launch shapes.  Not part of the GEMM path.
 *   src   device, 16-byte aligned, at least `bytes` readable
 *   bytes a positive multiple of 1024
 *   sink  device, 4-byte aligned, sink_bytes >= grid * waves * 4
 *   grid in [1, 65535] workgroups of 64 * waves threads, waves in
 *   {1, 2, 4, 8, 16}, depth in {1, 2, 4, 8}
 * Errors: W8_E_INVALID for any other argument; W8_E_HIP if the launch fails. */
w8_status w8_read_floor(const void *src, size_t bytes, void *sink, size_t sink_bytes, int grid,
                        int waves, int depth, w8_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* W8GEMM_H */
