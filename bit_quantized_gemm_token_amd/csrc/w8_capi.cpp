// C-ABI of the w8gemm library: argument validation, config resolution and
// kernel dispatch.  Nothing here allocates, frees or synchronizes on the
// quantize / GEMM path, so both can be captured into a HIP graph.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "w8_internal.hpp"

namespace w8 {

namespace {
thread_local std::string g_err;

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxK = 1 << 22;
constexpr int kMaxN = 1 << 24;

int nb_index(int nb) { return nb == 1 ? 0 : nb == 2 ? 1 : nb == 4 ? 2 : -1; }
int wk_index(int wk) {
  return wk == 1 ? 0 : wk == 2 ? 1 : wk == 4 ? 2 : wk == 8 ? 3 : wk == 16 ? 4 : -1;
}
int wn_index(int wn) { return wn == 1 ? 0 : wn == 2 ? 1 : wn == 4 ? 2 : wn == 8 ? 3 : -1; }
int u_index(int u) { return u == 1 ? 0 : u == 2 ? 1 : u == 4 ? 2 : -1; }
// weight layout 0 (row-major), 1, 2, 4, 8 (packed, K-steps per MFMA)
int lay_index(int l) { return l == 0 ? 0 : l == 1 ? 1 : l == 2 ? 2 : l == 4 ? 3 : l == 8 ? 4 : -1; }

// [fmt][mb-1][nb][wk][wn][unroll][swap][layout][xl][sk] -> launcher
struct InstanceIndex {
  GemmLaunchFn fn[3][2][3][5][4][3][2][5][4][2] = {};
  InstanceIndex() {
    int n = 0;
    const GemmInstance* p = gemm_instances(&n);
    for (int i = 0; i < n; ++i) {
      const GemmInstance& g = p[i];
      fn[g.fmt][g.mb - 1][nb_index(g.nb)][wk_index(g.wk)][wn_index(g.wn)][u_index(g.unroll)]
        [g.swap][lay_index(g.packed)][g.xl][g.sk] = g.fn;
    }
  }
};

const InstanceIndex& instance_index() {
  static const InstanceIndex idx;
  return idx;
}
}  // namespace

w8_status fail(w8_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

w8_status ok() {
  g_err.clear();
  return W8_OK;
}

std::string hip_msg(const char* what, hipError_t e) {
  return std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
}

const char* fmt_name(int fmt) {
  switch (fmt) {
    case W8_FP8_DYNAMIC: return "FP8_Dynamic";
    case W8_W8A8_INT8: return "W8A8_INT8";
    case W8_BLOCK_FP8: return "Block_FP8";
  }
  return "?";
}

int fmt_from_name(const std::string& s) {
  for (int f = 0; f < 3; ++f)
    if (s == fmt_name(f)) return f;
  return -1;
}

int ksteps_of(int fmt, int K) { return (K + kstep_of(fmt) - 1) / kstep_of(fmt); }

int layout_from_ldw(long long ldw) {
  if (ldw > 0) return 0;
  if (ldw == 0 || ldw == -1) return 1;
  if (ldw == -2 || ldw == -4 || ldw == -8) return (int)-ldw;
  return -1;
}

// Token rows one launch covers: 16 per MFMA block (two blocks) for row-major
// and plain packed weights, R = 16/T per group (two groups) for the
// K-segmented layouts; larger M runs as consecutive launches.
int launch_rows(int layout) { return 2 * layout_rows(layout); }

w8_status check_gemm_shape(int fmt, int M, int N, int K) {
  if (fmt < 0 || fmt > 2) return fail(W8_E_INVALID, "unknown format " + std::to_string(fmt));
  if (M < 1 || N < 1 || K < 1)
    return fail(W8_E_INVALID, "M, N and K must be positive (M=" + std::to_string(M) +
                                  ", N=" + std::to_string(N) + ", K=" + std::to_string(K) + ")");
  if (M > W8_MAX_M)
    return fail(W8_E_UNSUPPORTED, "M=" + std::to_string(M) + " is above the small-M window (" +
                                      std::to_string(W8_MAX_M) + "); use another backend");
  if (K % 16) return fail(W8_E_INVALID, "K must be a multiple of 16");
  if (fmt == W8_BLOCK_FP8 && K % W8_GROUP) return fail(W8_E_INVALID, "Block_FP8 needs K % 128 == 0");
  if (K > kMaxK) return fail(W8_E_INVALID, "K above 2^22");
  if (N > kMaxN) return fail(W8_E_INVALID, "N above 2^24");
  return W8_OK;
}

GemmLaunchFn find_instance(int fmt, int mb, const w8_cfg& c, int layout, int xl);
static int launch_mb(int M, int layout);

w8_status check_cfg(int fmt, int op, int M, int N, int K, const w8_cfg& c, int layout) {
  if (c.abi_version != W8_ABI_VERSION)
    return fail(W8_E_INVALID, "cfg.abi_version " + std::to_string(c.abi_version) + " != " +
                                  std::to_string(W8_ABI_VERSION));
  if (c.reserved[0]) return fail(W8_E_INVALID, "cfg.reserved must be zero");
  if (!layout_valid(layout)) return fail(W8_E_INVALID, "weight layout must be 0, 1, 2, 4 or 8");
  const int R = layout_rows(layout);
  if (nb_index(c.tile_n / R) < 0 || c.tile_n % R)
    return fail(W8_E_INVALID, layout > 1 ? "cfg.tile_n must be 1, 2 or 4 times the layout's " +
                                               std::to_string(R) + "-row block"
                                         : std::string("cfg.tile_n must be 16, 32 or 64"));
  if (layout > 1) {
    // K-segmented layouts: one wave along N, split-K; activations loaded by
    // each wave, or (the fused linear op) quantized into LDS by the kernel
    if (c.waves_n != 1 || c.grid != 0)
      return fail(W8_E_INVALID, "cfg: the K-segmented layouts run with waves_n 1 and grid 0");
    const bool fused = op == W8_OP_LINEAR && !c.quant_launch;
    if (c.x_lds != (fused ? 1 : 0))
      return fail(W8_E_INVALID, "cfg: on the K-segmented layouts x_lds is 1 exactly for the "
                                "fused linear op (quant_launch 0)");
    if (op == W8_OP_MOE || op == W8_OP_MOE_LINEAR)
      return fail(W8_E_INVALID, "the grouped GEMM runs on row-major and plain packed weights");
  }
  if (wk_index(c.waves_k) < 0) return fail(W8_E_INVALID, "cfg.waves_k must be 1, 2, 4, 8 or 16");
  if (wn_index(c.waves_n) < 0) return fail(W8_E_INVALID, "cfg.waves_n must be 1, 2, 4 or 8");
  if (c.waves_n > 1 && c.waves_k != 1)
    return fail(W8_E_INVALID, "cfg: waves_n > 1 needs waves_k == 1");
  if (c.x_lds != 0 && c.x_lds != 1) return fail(W8_E_INVALID, "cfg.x_lds must be 0 or 1");
  if (c.waves_n > 1 && !c.x_lds) return fail(W8_E_INVALID, "cfg: waves_n > 1 needs x_lds == 1");
  if (c.x_lds && c.waves_k > 8) return fail(W8_E_INVALID, "cfg: x_lds needs waves_k <= 8");
  if (op != W8_OP_GEMM && op != W8_OP_LINEAR && op != W8_OP_MOE && op != W8_OP_MOE_LINEAR)
    return fail(W8_E_INVALID, "unknown op");
  if (c.quant_launch != 0 && c.quant_launch != 1)
    return fail(W8_E_INVALID, "cfg.quant_launch must be 0 or 1");
  if (op != W8_OP_LINEAR && op != W8_OP_MOE_LINEAR && c.quant_launch)
    return fail(W8_E_INVALID, "cfg.quant_launch is for the linear ops only");
  // fused quantization: staged in LDS (x_lds 1), or for the Block_FP8
  // linear op also in the K loop (x_lds 0: each wave quantizes the 1x128
  // groups it loads)
  if ((op == W8_OP_LINEAR || op == W8_OP_MOE_LINEAR) && !c.quant_launch &&
      (c.x_lds ? c.waves_k > 4
               : (op != W8_OP_LINEAR || fmt != W8_BLOCK_FP8 || c.unroll != 1 ||
                  c.tile_n > 32 || c.waves_k < 2 || c.waves_k > 8)))
    return fail(W8_E_INVALID,
                "cfg: fused quantization (quant_launch == 0) needs x_lds == 1 and waves_k <= 4, "
                "or for the Block_FP8 linear op x_lds == 0 (quantized in the K loop) with "
                "tile_n 16 or 32, unroll 1 and waves_k 2, 4 or 8");
  if (u_index(c.unroll) < 0) return fail(W8_E_INVALID, "cfg.unroll must be 1, 2 or 4");
  if ((c.tile_n / R) * c.unroll > 4)
    return fail(W8_E_INVALID, "cfg: (blocks per wave) * unroll must be at most 4");
  if (!is_pow2(c.split_k) || c.split_k > W8_MAX_SPLIT_K)
    return fail(W8_E_INVALID, "cfg.split_k must be a power of two in [1, 256], got " +
                                  std::to_string(c.split_k));
  if (c.swap_ab != 0 && c.swap_ab != 1) return fail(W8_E_INVALID, "cfg.swap_ab must be 0 or 1");
  const long long ntiles = tiles_of(N, c);
  const long long iters = ntiles * layout_spans(fmt, K, layout);
  if (c.grid < 0) return fail(W8_E_INVALID, "cfg.grid must be >= 0");
  if (c.grid > 0) {
    if (c.split_k != 1) return fail(W8_E_INVALID, "cfg: stream-K (grid > 0) needs split_k == 1");
    if (c.tile_n != 16 || c.unroll > 2)
      return fail(W8_E_INVALID, "cfg: stream-K (grid > 0) is compiled for tile_n 16 with "
                                "unroll 1 or 2 only");
    if (c.grid > iters)
      return fail(W8_E_INVALID, "cfg.grid " + std::to_string(c.grid) +
                                    " exceeds the (tile, K-step) iterations (" +
                                    std::to_string(iters) + ")");
  }
  if (c.x_lds) {
    // K-steps (spans) of a workgroup x token blocks of one launch x 1 KiB chunks
    const long long ks = layout_spans(fmt, K, layout);
    const long long seg = c.grid > 0 ? std::min(ks, (iters + c.grid - 1) / c.grid)
                                     : (ks + c.split_k - 1) / c.split_k;
    const long long chunks =
        seg * launch_mb(std::min(M, launch_rows(layout)), layout) * (kstep_of(fmt) / 64);
    if (chunks > kXlChunks)
      return fail(W8_E_INVALID, "cfg: x_lds needs the activations of a workgroup's K range in "
                                "64 KiB (" + std::to_string(chunks) + " KiB here)");
  }
  if ((c.split_k > 1 || c.grid > 0) && ntiles > kSplitKMaxTiles)
    return fail(W8_E_INVALID, "split_k > 1 and grid > 0 support at most " +
                                  std::to_string(kSplitKMaxTiles) + " output tiles (N <= " +
                                  std::to_string((long long)kSplitKMaxTiles * c.tile_n * c.waves_n) +
                                  ")");
  // one-dimensional grid: the launch's total thread count must fit in 32 bits
  const long long wgs = c.grid > 0 ? c.grid : ntiles * c.split_k;
  const long long threads = wgs * 64 * c.waves_k * c.waves_n;
  if (threads > 0xFFFFFFFFLL)
    return fail(W8_E_INVALID, "cfg: (workgroups x waves x 64) threads exceed 2^32 - 1");
  if (op == W8_OP_GEMM || op == W8_OP_LINEAR) {
    // a compiled kernel for each launch of the call (all of `rows` token
    // rows but a shorter last one)
    const int xl = (op == W8_OP_LINEAR && !c.quant_launch) ? (c.x_lds ? 2 : 3) : c.x_lds;
    const int rows = launch_rows(layout);
    const int last = M % rows ? M % rows : rows;
    if (!find_instance(fmt, launch_mb(std::min(M, rows), layout), c, layout, xl) ||
        !find_instance(fmt, launch_mb(last, layout), c, layout, xl))
      return fail(W8_E_INVALID, "no compiled kernel for this config and weight layout");
  }
  return W8_OK;
}

int tiles_of(int N, const w8_cfg& c) {
  const int cols = c.tile_n * c.waves_n;
  return (N + cols - 1) / cols;
}

int partial_slots(int fmt, int N, int K, const w8_cfg& c) {
  if (c.grid > 0) return stream_k_slots(tiles_of(N, c), ksteps_of(fmt, K), c.grid);
  return c.split_k;
}

// Blocks of token rows in one launch (the kernel's MB).
static int launch_mb(int M, int layout) {
  const int R = layout_rows(layout);
  return std::min(2, (M + R - 1) / R);
}

static size_t gemm_ws_bytes(int fmt, int M, int N, int K, const w8_cfg& c, int layout) {
  if (c.split_k <= 1 && c.grid <= 0) return 0;
  const int ntiles = tiles_of(N, c);
  return ws_counter_bytes(ntiles) +
         ws_partial_bytes(ntiles, partial_slots(fmt, N, K, c),
                          c.waves_n * c.tile_n / layout_rows(layout), launch_mb(M, layout));
}

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

LinearWs linear_ws(int fmt, int M, int N, int K, const w8_cfg& c, int layout) {
  LinearWs w;
  w.ldq = (K + 15) / 16 * 16;
  // past the arrival counters even when this config shares no tile: another
  // call on the same workspace relies on their values
  w.codes = round256(std::max(gemm_ws_bytes(fmt, M, N, K, c, layout), ws_counter_bytes(0)));
  w.scales = w.codes + round256((size_t)M * w.ldq);
  const size_t nsx = fmt == W8_BLOCK_FP8 ? (size_t)M * (K / W8_GROUP) : (size_t)M;
  w.total = w.scales + round256(nsx * 4);
  return w;
}

size_t workspace_bytes(int fmt, int op, int M, int N, int K, const w8_cfg& c, int layout) {
  if (op == W8_OP_LINEAR && c.quant_launch) return linear_ws(fmt, M, N, K, c, layout).total;
  return gemm_ws_bytes(fmt, M, N, K, c, layout);
}

// Default config (used when the table has no entry for the shape).  It
// follows the rule of thumb the page quotes for vLLM's Block_FP8 backend --
// Swap-AB below 32 tokens -- for every format, and picks the smallest
// split_k that gives at least two workgroups per compute unit while every
// wave keeps at least one full stage of K-steps.  The fused linear op stages
// activations in LDS (x_lds), so it doubles split_k further until a
// workgroup's K range of activations fits.  The K-segmented layouts take one
// block per wave, two K-waves, and the linear op a quantize launch.
w8_cfg make_default_cfg(int fmt, int op, int M, int N, int K, int layout) {
  w8_cfg c;
  std::memset(&c, 0, sizeof c);
  c.abi_version = W8_ABI_VERSION;
  c.tile_n = 16;
  c.waves_k = 4;
  c.waves_n = 1;
  c.unroll = 2;
  c.swap_ab = M < 32 ? 1 : 0;
  if (layout > 1) {
    const int R = layout_rows(layout);
    const int spans = layout_spans(fmt, K, layout);
    c.tile_n = R;
    c.waves_k = 2;
    c.swap_ab = 1;
    int s = 1;
    while (s < W8_MAX_SPLIT_K && (long long)((N + R - 1) / R) * s < 256 &&
           spans / (2 * s) >= c.waves_k * c.unroll)
      s *= 2;
    c.split_k = s;
    if (op == W8_OP_LINEAR) c.quant_launch = 1;
    return c;
  }
  const int ntiles = (N + 15) / 16;
  const int T = ksteps_of(fmt, K);
  int s = 1;
  while (s < W8_MAX_SPLIT_K && (long long)ntiles * s < 512 &&
         T / (2 * s) >= c.waves_k * c.unroll)
    s *= 2;
  c.split_k = s;
  if (op == W8_OP_LINEAR) {
    c.x_lds = 1;
    const long long per_step = (long long)((M + 15) / 16) * (kstep_of(fmt) / 64);
    while (c.split_k < W8_MAX_SPLIT_K && (T + c.split_k - 1) / c.split_k * per_step > kXlChunks)
      c.split_k *= 2;
  }
  return c;
}

w8_status check_device() {
  static std::atomic<int> state[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("hipGetDevice", e));
  if (dev < 0 || dev >= 64) return fail(W8_E_UNSUPPORTED, "device index out of range");
  int st = state[dev].load();
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("hipGetDeviceProperties", e));
    st = std::strncmp(prop.gcnArchName, kArch, std::strlen(kArch)) == 0 ? 1 : 2;
    state[dev].store(st);
  }
  if (st != 1) return fail(W8_E_UNSUPPORTED, "this library is built for gfx950 only");
  return W8_OK;
}

GemmLaunchFn find_instance(int fmt, int mb, const w8_cfg& c, int layout, int xl) {
  const int nb = c.tile_n / layout_rows(layout);
  if (mb < 1 || mb > 2 || nb_index(nb) < 0 || wk_index(c.waves_k) < 0 ||
      wn_index(c.waves_n) < 0 || u_index(c.unroll) < 0 || lay_index(layout) < 0 ||
      c.swap_ab < 0 || c.swap_ab > 1 || xl < 0 || xl > 3)
    return nullptr;
  return instance_index().fn[fmt][mb - 1][nb_index(nb)][wk_index(c.waves_k)][wn_index(c.waves_n)]
                            [u_index(c.unroll)][c.swap_ab][lay_index(layout)][xl]
                            [c.grid > 0 ? 1 : 0];
}

w8_status launch_gemm_call(const GemmCall& g, const w8_cfg& c, hipStream_t s) {
  const int rows = launch_rows(g.layout);
  if (g.M > rows) {
    // consecutive launches of `rows` token rows each (K-segmented layouts;
    // they share the workspace, in stream order)
    for (int m0 = 0; m0 < g.M; m0 += rows) {
      GemmCall p = g;
      p.M = std::min(rows, g.M - m0);
      if (g.x) {  // fused quantization: bf16 rows, scales computed by the kernel
        p.x = static_cast<const uint16_t*>(g.x) + (long long)m0 * g.ldx;
      } else {
        p.xq = static_cast<const uint8_t*>(g.xq) + (long long)m0 * g.ldq;
        p.sx = g.sx + (long long)m0 * (g.fmt == W8_BLOCK_FP8 ? g.K / W8_GROUP : 1);
      }
      p.out = static_cast<char*>(g.out) + (long long)m0 * g.ldo * (g.out_mode ? 4 : 2);
      const w8_status st = launch_gemm_call(p, c, s);
      if (st) return st;
    }
    return W8_OK;
  }
  const int mb = launch_mb(g.M, g.layout);
  GemmLaunchFn fn = find_instance(g.fmt, mb, c, g.layout, g.x ? (c.x_lds ? 2 : 3) : c.x_lds);
  if (!fn) return fail(W8_E_INVALID, "no compiled kernel for this config");
  const int ntiles = tiles_of(g.N, c);
  const int T = layout_segments(g.layout);
  GemmArgs a;
  a.xq = static_cast<const uint8_t*>(g.x ? g.x : g.xq);  // fused: bf16 activations
  a.sx = g.sx;
  a.wq = static_cast<const uint8_t*>(g.wq);
  a.sw = g.sw;
  a.out = g.out;
  a.ldq = g.x ? g.ldx : g.ldq;
  a.ldw = g.layout ? 0 : g.ldw;
  a.ldo = g.ldo;
  a.M = g.M;
  a.N = g.N;
  a.K = g.K;
  // the K loop's steps: K-steps, or spans of T of them
  a.ksteps = layout_spans(g.fmt, g.K, g.layout);
  a.kfull = g.K / kstep_of(g.fmt) / T;
  a.split_k = c.split_k;
  a.split_shift = __builtin_ctz((unsigned)c.split_k);
  a.grid = c.grid;
  a.slots = partial_slots(g.fmt, g.N, g.K, c);
  a.ntiles = ntiles;
  a.sgroups = g.fmt == W8_BLOCK_FP8 ? g.K / W8_GROUP : 0;
  a.out_mode = g.out_mode;
  a.counters = nullptr;
  a.part = nullptr;
  if (c.split_k > 1 || c.grid > 0) {
    a.counters = static_cast<unsigned int*>(g.ws);
    a.part = static_cast<char*>(g.ws) + ws_counter_bytes(ntiles);
  }
  const unsigned wgs = c.grid > 0 ? (unsigned)c.grid : (unsigned)(ntiles * c.split_k);
  hipError_t e = fn(a, dim3(wgs), dim3(64 * c.waves_k * c.waves_n), s);
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("GEMM launch", e));
  return W8_OK;
}

w8_status launch_linear_call(const GemmCall& g, const w8_cfg& c, hipStream_t s) {
  if (!c.quant_launch) return launch_gemm_call(g, c, s);
  // quantize into the workspace, then the GEMM on the codes
  const LinearWs w = linear_ws(g.fmt, g.M, g.N, g.K, c, g.layout);
  char* base = static_cast<char*>(g.ws);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + w.codes);
  float* sx = reinterpret_cast<float*>(base + w.scales);
  QuantActArgs q{static_cast<const uint16_t*>(g.x), xq, sx, g.ldx, w.ldq, g.M, g.K};
  hipError_t e = launch_quantize_act(g.fmt, q, s);
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("quantize_act launch", e));
  GemmCall gg = g;
  gg.xq = xq;
  gg.ldq = w.ldq;
  gg.sx = sx;
  gg.x = nullptr;
  gg.ldx = 0;
  gg.ws_bytes = w.codes;
  return launch_gemm_call(gg, c, s);
}

}  // namespace w8

using namespace w8;

namespace {

w8_status gemm_entry(int fmt, int M, int N, int K, const void* xq, int64_t ldq,
                     const float* sx, const void* wq, int64_t ldw, const float* sw, void* out,
                     int64_t ldo, const w8_cfg* cfg, void* ws, size_t ws_bytes,
                     w8_stream stream, int out_mode) {
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!xq || !sx || !wq || !sw || !out) return fail(W8_E_INVALID, "null device pointer");
  if (!aligned(xq, 16) || !aligned(wq, 16))
    return fail(W8_E_INVALID, "xq and wq must be 16-byte aligned");
  const int layout = layout_from_ldw(ldw);  // ldw <= 0: packed weights
  if (ldq < K || ldq % 16 || layout < 0 || (!layout && (ldw < K || ldw % 16)))
    return fail(W8_E_INVALID,
                "ldq must be >= K and a multiple of 16; ldw must be >= K and a multiple of 16 "
                "(row-major weights), 0 (packed) or -2, -4, -8 (K-segmented packed)");
  if (ldo < N) return fail(W8_E_INVALID, "output leading dimension must be >= N");
  if (!aligned(sx, 4) || !aligned(sw, 4) || !aligned(out, out_mode ? 4 : 2))
    return fail(W8_E_INVALID, "misaligned scale or output pointer");
  w8_cfg c;
  if (cfg) {
    c = *cfg;
    st = check_cfg(fmt, W8_OP_GEMM, M, N, K, c, layout);
    if (st) return st;
  } else {
    c = resolve_cfg(fmt, W8_OP_GEMM, M, N, K, layout, nullptr);
  }
  const size_t need = workspace_bytes(fmt, W8_OP_GEMM, M, N, K, c, layout);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(W8_E_WORKSPACE, "workspace of " + std::to_string(need) + " bytes needed, got " +
                                      std::to_string(ws ? ws_bytes : 0));
    if (!aligned(ws, 16)) return fail(W8_E_INVALID, "workspace must be 16-byte aligned");
  }
  st = check_device();
  if (st) return st;
  GemmCall g{fmt, M, N, K, xq, ldq, sx, wq, ldw, sw, out, ldo, out_mode, ws, ws_bytes, layout,
             nullptr, 0};
  st = launch_gemm_call(g, c, static_cast<hipStream_t>(stream));
  if (st) return st;
  return ok();
}

// ------------------------------------------------ the no-allocation entry --
// w8_gemm_w8a8_noalloc keeps the split-K workspace (arrival counters, then
// partials) in this file-scope device array instead of a caller's buffer.
// The loader zero-fills it on each device; every call leaves its arrival
// counters at multiples of 256 (the split-K counters rise by 256 a launch,
// the stream-K ones return to zero), and the partials are written before
// they are read, so nothing needs clearing between calls.  Its host-side name is not a device
// address: the address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)16 << 20;  // 2 MiB of counters + 14 MiB of partials
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

w8_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("hipGetDevice", e));
  if (dev < 0 || dev >= 64) return fail(W8_E_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(W8_E_HIP, hip_msg("hipGetSymbolAddress(scratch)", e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return W8_OK;
}

}  // namespace

extern "C" {

int w8_abi_version(void) { return W8_ABI_VERSION; }

const char* w8_status_string(w8_status s_in) {
  const int s = raw_enum(s_in);
  switch (s) {
    case W8_OK: return "W8_OK";
    case W8_E_INVALID: return "W8_E_INVALID";
    case W8_E_UNSUPPORTED: return "W8_E_UNSUPPORTED";
    case W8_E_WORKSPACE: return "W8_E_WORKSPACE";
    case W8_E_TABLE_FORMAT: return "W8_E_TABLE_FORMAT";
    case W8_E_IO: return "W8_E_IO";
    case W8_E_HIP: return "W8_E_HIP";
    case W8_E_VALIDATION: return "W8_E_VALIDATION";
    case W8_E_NOT_FOUND: return "W8_E_NOT_FOUND";
  }
  return "W8_E_UNKNOWN";
}

const char* w8_last_error(void) { return g_err.c_str(); }

w8_status w8_quantize_act(w8_fmt fmt_in, int M, int K, const void* x, int64_t ldx, void* xq,
                          int64_t ldq, float* sx, w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_gemm_shape(fmt, M, 1, K);
  if (st) return st;
  if (!x || !xq || !sx) return fail(W8_E_INVALID, "null device pointer");
  if (!aligned(x, 16) || ldx % 8 || ldx < K)
    return fail(W8_E_INVALID, "x must be 16-byte aligned with ldx >= K and ldx % 8 == 0");
  if (!aligned(xq, 16) || ldq % 16 || ldq < K)
    return fail(W8_E_INVALID, "xq must be 16-byte aligned with ldq >= K and ldq % 16 == 0");
  if (!aligned(sx, 4)) return fail(W8_E_INVALID, "sx must be 4-byte aligned");
  st = check_device();
  if (st) return st;
  QuantActArgs a{static_cast<const uint16_t*>(x), static_cast<uint8_t*>(xq), sx, ldx, ldq, M, K};
  hipError_t e = launch_quantize_act(fmt, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("quantize_act launch", e));
  return ok();
}

w8_status w8_quantize_weight(w8_fmt fmt_in, int N, int K, const float* w, int64_t ldw, void* wq,
                             int64_t ldq, float* sw, w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  if (fmt != W8_FP8_DYNAMIC && fmt != W8_BLOCK_FP8)
    return fail(W8_E_INVALID, "weight quantization is defined for FP8_Dynamic and Block_FP8");
  if (N < 1 || K < 1 || N > kMaxN || K > kMaxK) return fail(W8_E_INVALID, "bad N or K");
  if (!w || !wq || !sw) return fail(W8_E_INVALID, "null device pointer");
  if (ldw < K || ldq < K) return fail(W8_E_INVALID, "leading dimensions must be >= K");
  if (!aligned(w, 4) || !aligned(sw, 4)) return fail(W8_E_INVALID, "misaligned w or sw");
  w8_status st = check_device();
  if (st) return st;
  QuantWeightArgs a{w, static_cast<uint8_t*>(wq), sw, ldw, ldq, N, K};
  hipError_t e = launch_quantize_weight(fmt, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("quantize_weight launch", e));
  return ok();
}

w8_status w8_workspace_size(w8_fmt fmt_in, w8_op op_in, int M, int N, int K, int layout,
                            const w8_cfg* cfg, size_t* bytes) {
  const int fmt = raw_enum(fmt_in);
  const int op = raw_enum(op_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!bytes) return fail(W8_E_INVALID, "null output pointer");
  if (op != W8_OP_GEMM && op != W8_OP_LINEAR) return fail(W8_E_INVALID, "unknown op");
  if (!layout_valid(layout)) return fail(W8_E_INVALID, "weight layout must be 0, 1, 2, 4 or 8");
  w8_cfg c;
  if (cfg) {
    c = *cfg;
    st = check_cfg(fmt, op, M, N, K, c, layout);
    if (st) return st;
  } else {
    c = resolve_cfg(fmt, op, M, N, K, layout, nullptr);
  }
  *bytes = workspace_bytes(fmt, op, M, N, K, c, layout);
  return ok();
}

w8_status w8_packed_weight_size(w8_fmt fmt_in, int N, int K, int layout, size_t* bytes) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_gemm_shape(fmt, 1, N, K);
  if (st) return st;
  if (!bytes) return fail(W8_E_INVALID, "null output pointer");
  if (layout != 1 && layout != 2 && layout != 4 && layout != 8)
    return fail(W8_E_INVALID, "packed layout must be 1, 2, 4 or 8");
  *bytes = packed_weight_bytes(fmt, N, K, layout);
  return ok();
}

w8_status w8_pack_weight(w8_fmt fmt_in, int N, int K, const void* wq, int64_t ldw, void* wp,
                         int layout, w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_gemm_shape(fmt, 1, N, K);
  if (st) return st;
  if (layout != 1 && layout != 2 && layout != 4 && layout != 8)
    return fail(W8_E_INVALID, "packed layout must be 1, 2, 4 or 8");
  if (!wq || !wp) return fail(W8_E_INVALID, "null device pointer");
  if (!aligned(wq, 16) || !aligned(wp, 16) || ldw < K || ldw % 16)
    return fail(W8_E_INVALID, "wq and wp must be 16-byte aligned, ldw >= K and ldw % 16 == 0");
  st = check_device();
  if (st) return st;
  hipError_t e = launch_pack_weight(fmt, static_cast<const uint8_t*>(wq), ldw, N, K,
                                    static_cast<uint8_t*>(wp), layout,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("pack_weight launch", e));
  return ok();
}

w8_status w8_gemm_w8a8(w8_fmt fmt_in, int M, int N, int K, const void* xq, int64_t ldq,
                       const float* sx, const void* wq, int64_t ldw, const float* sw, void* y,
                       int64_t ldy, const w8_cfg* cfg, void* ws, size_t ws_bytes,
                       w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  return gemm_entry(fmt, M, N, K, xq, ldq, sx, wq, ldw, sw, y, ldy, cfg, ws, ws_bytes, stream, 0);
}

w8_status w8_gemm_w8a8_noalloc(w8_fmt fmt_in, int M, int N, int K, const void* xq, int64_t ldq,
                               const float* sx, const void* wq, int64_t ldw, const float* sw,
                               void* y, int64_t ldy, const w8_cfg* cfg, w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  const int layout = layout_from_ldw(ldw);
  if (layout < 0) return fail(W8_E_INVALID, "ldw must be > 0, 0, -2, -4 or -8");
  w8_cfg c;
  if (cfg) {
    c = *cfg;
    st = check_cfg(fmt, W8_OP_GEMM, M, N, K, c, layout);
    if (st) return st;
  } else {
    c = resolve_cfg(fmt, W8_OP_GEMM, M, N, K, layout, nullptr);
  }
  const size_t need = workspace_bytes(fmt, W8_OP_GEMM, M, N, K, c, layout);
  if (need > kScratchBytes)
    return fail(W8_E_WORKSPACE, "the config needs " + std::to_string(need) +
                                    " bytes of workspace; the no-allocation entry point has " +
                                    std::to_string(kScratchBytes) +
                                    " (use w8_gemm_w8a8 with a workspace, or a config with less "
                                    "split_k)");
  st = check_device();
  if (st) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st) return st;
  }
  return gemm_entry(fmt, M, N, K, xq, ldq, sx, wq, ldw, sw, y, ldy, &c, ws,
                    need > 0 ? kScratchBytes : 0, stream, 0);
}

w8_status w8_gemm_w8a8_acc(w8_fmt fmt_in, int M, int N, int K, const void* xq, int64_t ldq,
                           const float* sx, const void* wq, int64_t ldw, const float* sw,
                           void* acc, int64_t ldacc, const w8_cfg* cfg, void* ws,
                           size_t ws_bytes, w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  return gemm_entry(fmt, M, N, K, xq, ldq, sx, wq, ldw, sw, acc, ldacc, cfg, ws, ws_bytes, stream,
                    1);
}

w8_status w8_linear(w8_fmt fmt_in, int M, int N, int K, const void* x, int64_t ldx, const void* wq,
                    int64_t ldw, const float* sw, void* y, int64_t ldy, const w8_cfg* cfg,
                    void* ws, size_t ws_bytes, w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!x || !wq || !sw || !y) return fail(W8_E_INVALID, "null device pointer");
  if (!aligned(x, 16) || ldx % 8 || ldx < K)
    return fail(W8_E_INVALID, "x must be 16-byte aligned with ldx >= K and ldx % 8 == 0");
  if (!aligned(wq, 16)) return fail(W8_E_INVALID, "wq must be 16-byte aligned");
  const int layout = layout_from_ldw(ldw);
  if (layout < 0 || (!layout && (ldw < K || ldw % 16)))
    return fail(W8_E_INVALID, "ldw must be >= K and a multiple of 16 (row-major weights), 0 "
                              "(packed) or -2, -4, -8 (K-segmented packed)");
  if (ldy < N) return fail(W8_E_INVALID, "output leading dimension must be >= N");
  if (!aligned(sw, 4) || !aligned(y, 2)) return fail(W8_E_INVALID, "misaligned sw or y");
  w8_cfg c;
  if (cfg) {
    c = *cfg;
    st = check_cfg(fmt, W8_OP_LINEAR, M, N, K, c, layout);
    if (st) return st;
  } else {
    c = resolve_cfg(fmt, W8_OP_LINEAR, M, N, K, layout, nullptr);
  }
  const size_t need = workspace_bytes(fmt, W8_OP_LINEAR, M, N, K, c, layout);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(W8_E_WORKSPACE, "workspace of " + std::to_string(need) + " bytes needed, got " +
                                      std::to_string(ws ? ws_bytes : 0));
    if (!aligned(ws, 16)) return fail(W8_E_INVALID, "workspace must be 16-byte aligned");
  }
  st = check_device();
  if (st) return st;
  GemmCall g{fmt, M, N, K, nullptr, 0, nullptr, wq, ldw, sw, y, ldy, 0, ws, ws_bytes, layout,
             x, ldx};
  st = launch_linear_call(g, c, static_cast<hipStream_t>(stream));
  if (st) return st;
  return ok();
}

w8_status w8_validate_config(w8_fmt fmt_in, w8_op op_in, int M, int N, int K, int layout,
                             const w8_cfg* cfg) {
  const int fmt = raw_enum(fmt_in);
  const int op = raw_enum(op_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!cfg) return fail(W8_E_INVALID, "null cfg");
  if (op == W8_OP_MOE || op == W8_OP_MOE_LINEAR)
    return fail(W8_E_INVALID, "grouped configs: w8_moe_validate_config");
  st = check_cfg(fmt, op, M, N, K, *cfg, layout);
  if (st) return st;
  return ok();
}

w8_status w8_default_config(w8_fmt fmt_in, w8_op op_in, int M, int N, int K, int layout, w8_cfg* out) {
  const int fmt = raw_enum(fmt_in);
  const int op = raw_enum(op_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!out) return fail(W8_E_INVALID, "null output pointer");
  if (op != W8_OP_GEMM && op != W8_OP_LINEAR) return fail(W8_E_INVALID, "unknown op");
  if (!layout_valid(layout)) return fail(W8_E_INVALID, "weight layout must be 0, 1, 2, 4 or 8");
  *out = make_default_cfg(fmt, op, M, N, K, layout);
  return ok();
}

w8_status w8_resolve_config(w8_fmt fmt_in, w8_op op_in, int M, int N, int K, int layout, w8_cfg* out,
                            int* from_table) {
  const int fmt = raw_enum(fmt_in);
  const int op = raw_enum(op_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!out) return fail(W8_E_INVALID, "null output pointer");
  if (op != W8_OP_GEMM && op != W8_OP_LINEAR) return fail(W8_E_INVALID, "unknown op");
  if (!layout_valid(layout)) return fail(W8_E_INVALID, "weight layout must be 0, 1, 2, 4 or 8");
  int hit = 0;
  *out = resolve_cfg(fmt, op, M, N, K, layout, &hit);
  if (from_table) *from_table = hit;
  return ok();
}

}  // extern "C"
