// C-ABI of the MoE grouped GEMM (ai-radar.it, "Helion nel backend vLLM",
// paragraph 9: MoE models, whose MoE backend becomes the main optimization
// target, are the work's next stated goal).  One launch covers every expert:
// grid.y is the expert, and each expert runs the GEMM family's kernel on the
// token rows routed to it (gathered through a row-index list), its own
// weights and weight scales, and its own shared-tile workspace.
#include <algorithm>
#include <cstring>
#include <string>

#include "w8_internal.hpp"

namespace w8 {
namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
int nb_index(int nb) { return nb == 1 ? 0 : nb == 2 ? 1 : nb == 4 ? 2 : -1; }
int wk_index(int wk) {
  return wk == 1 ? 0 : wk == 2 ? 1 : wk == 4 ? 2 : wk == 8 ? 3 : wk == 16 ? 4 : -1;
}
int wn_index(int wn) { return wn == 1 ? 0 : wn == 2 ? 1 : wn == 4 ? 2 : wn == 8 ? 3 : -1; }
int u_index(int u) { return u == 1 ? 0 : u == 2 ? 1 : u == 4 ? 2 : -1; }

struct MoeIndex {
  MoeLaunchFn fn[3][2][3][5][4][3][2][2][3][2] = {};
  MoeIndex() {
    int n = 0;
    const MoeInstance* p = moe_instances(&n);
    for (int i = 0; i < n; ++i) {
      const MoeInstance& g = p[i];
      fn[g.fmt][g.mb - 1][nb_index(g.nb)][wk_index(g.wk)][wn_index(g.wn)][u_index(g.unroll)]
        [g.swap][g.packed][g.xl][g.sk] = g.fn;
    }
  }
};

const MoeIndex& moe_index() {
  static const MoeIndex idx;
  return idx;
}

// in_kernel: quantization inside the kernel (bf16 activations, staged in
// LDS: needs x_lds).
MoeLaunchFn moe_fn(int fmt, int max_m, int packed, const w8_cfg& c, bool in_kernel) {
  if (c.x_lds > 1 || (in_kernel && !c.x_lds)) return nullptr;
  return moe_index().fn[fmt][(max_m + 15) / 16 - 1][nb_index(c.tile_n / 16)][wk_index(c.waves_k)]
                       [wn_index(c.waves_n)][u_index(c.unroll)][c.swap_ab][packed]
                       [in_kernel ? 2 : c.x_lds][c.grid > 0 ? 1 : 0];
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Bytes between two experts' partials (0 when no tile is shared).
size_t part_stride(int fmt, int max_m, int N, int K, const w8_cfg& c) {
  if (c.split_k <= 1 && c.grid <= 0) return 0;
  return round256(ws_partial_bytes(tiles_of(N, c), partial_slots(fmt, N, K, c),
                                   c.waves_n * c.tile_n / 16, (max_m + 15) / 16));
}

// w8_moe_linear with quant_launch: the T tokens' codes and scales follow the
// shared-tile region of the workspace (past the arrival counters even when
// no tile is shared: another call on the workspace relies on their values).
struct MoeQuantWs {
  size_t codes, scales, total;
  long long ldq;
};
MoeQuantWs moe_quant_ws(int fmt, int T, int K, size_t shared_bytes) {
  MoeQuantWs w;
  w.ldq = (K + 15) / 16 * 16;
  w.codes = round256(std::max(shared_bytes, ws_counter_bytes(0)));
  w.scales = w.codes + round256((size_t)T * w.ldq);
  const size_t nsx = fmt == W8_BLOCK_FP8 ? (size_t)T * (K / W8_GROUP) : (size_t)T;
  w.total = w.scales + round256(nsx * 4);
  return w;
}

size_t shared_ws_bytes(int fmt, int E, int max_m, int N, int K, const w8_cfg& c) {
  const size_t stride = part_stride(fmt, max_m, N, K, c);
  return stride ? ws_counter_bytes(0) + (size_t)E * stride : 0;
}

}  // namespace

// A config of the GEMM family (its rules at M = max_m; fused: the rules of
// w8_moe_linear's op) that has a compiled grouped instance -- the fused
// kernel, or with quant_launch the kernel on quantized activations -- and
// whose shared tiles fit the counter region.
w8_status check_moe_cfg(int fmt, int E, int max_m, int N, int K, int packed, const w8_cfg& c,
                        bool fused) {
  if (packed != 0 && packed != 1)
    return fail(W8_E_INVALID, "the grouped GEMM runs on row-major and plain packed weights");
  w8_status st = check_cfg(fmt, fused ? W8_OP_MOE_LINEAR : W8_OP_GEMM, max_m, N, K, c, packed);
  if (st) return st;
  const bool in_kernel = fused && !c.quant_launch;
  if (!moe_fn(fmt, max_m, packed, c, in_kernel))
    return fail(W8_E_INVALID,
                in_kernel ? "cfg: the fused grouped GEMM is compiled for (waves_k, waves_n, "
                            "x_lds) in {(1, 4|8, 1)}"
                          : "cfg: the grouped GEMM is compiled for (waves_k, waves_n, x_lds) in "
                            "{(1|2|4|8, 1, 0), (1, 2|4|8, 1)}");
  if ((c.split_k > 1 || c.grid > 0) && (long long)E * tiles_of(N, c) > kSplitKMaxTiles)
    return fail(W8_E_INVALID, "cfg: shared tiles need experts x tiles <= " +
                                  std::to_string(kSplitKMaxTiles));
  return W8_OK;
}

size_t moe_ws_bytes(int fmt, int E, int T, int max_m, int N, int K, const w8_cfg& c) {
  const size_t shared = shared_ws_bytes(fmt, E, max_m, N, K, c);
  return c.quant_launch ? moe_quant_ws(fmt, T, K, shared).total : shared;
}

// Default.  Measured on 128-expert top-8 layers (1536 x 2048 and 2048 x 768)
// at 1 to 32 tokens, the fastest grouped configs are small workgroups that
// each own 32 output columns of one expert, with no split and activations
// loaded in the K loop: the launch has workgroups to spare across the active
// experts, and a routed expert holds only a token or two.  Two K-waves of
// two K-steps each help when at most 2 tokens are routed.  If that config is
// invalid for the shape, the cost model's fastest valid config for a GEMM
// whose N spans the experts a call can reach -- min(E, 8 T) of them -- is
// used.
w8_cfg moe_fallback_cfg(int fmt, int E, int T, int max_m, int N, int K, int packed,
                        bool fused) {
  if (fused) {  // quantize in a launch of its own, then the grouped kernel
    w8_cfg c = moe_fallback_cfg(fmt, E, T, max_m, N, K, packed, false);
    c.quant_launch = 1;
    return c;
  }
  w8_cfg d;
  std::memset(&d, 0, sizeof d);
  d.abi_version = W8_ABI_VERSION;
  d.tile_n = 32;
  d.waves_k = T <= 2 ? 2 : 1;
  d.waves_n = 1;
  d.unroll = T <= 2 ? 2 : 1;
  d.split_k = 1;
  if (check_moe_cfg(fmt, E, max_m, N, K, packed, d, false) == W8_OK) return d;
  const long long reach = std::min<long long>(E, 8LL * T);
  const int n_eff = (int)std::min<long long>((long long)N * reach, 1 << 24);
  for (const auto& pc : rank_configs(fmt, W8_OP_GEMM, max_m, n_eff, K, packed, W8_MAX_SPLIT_K, 0))
    if (check_moe_cfg(fmt, E, max_m, N, K, packed, pc.second, false) == W8_OK) return pc.second;
  w8_cfg c;
  std::memset(&c, 0, sizeof c);
  c.abi_version = W8_ABI_VERSION;
  c.tile_n = 16;
  c.waves_k = 4;
  c.waves_n = 1;
  c.unroll = 1;
  c.split_k = 1;
  return c;
}

namespace {

// The config for cfg == NULL: the table entry for (fmt, moe or moe_linear,
// layout, T, N, K) if valid here, else the fallback.
w8_cfg moe_default_cfg(int fmt, int E, int T, int max_m, int N, int K, int packed, bool fused,
                       int* from_table) {
  w8_cfg c;
  if (from_table) *from_table = 0;
  if (w8_lookup_config((w8_fmt)fmt, fused ? W8_OP_MOE_LINEAR : W8_OP_MOE, T, N, K, packed, &c,
                       nullptr) == W8_OK &&
      check_moe_cfg(fmt, E, max_m, N, K, packed, c, fused) == W8_OK) {
    if (from_table) *from_table = 1;
    return c;
  }
  if (fused) {  // the quantized-activation op's config after a quantize launch
    c = moe_default_cfg(fmt, E, T, max_m, N, K, packed, false, nullptr);
    c.quant_launch = 1;
    return c;
  }
  return moe_fallback_cfg(fmt, E, T, max_m, N, K, packed, false);
}

w8_status check_moe_shape(int fmt, int E, int T, int N, int K, int max_m) {
  w8_status st = check_gemm_shape(fmt, max_m, N, K);
  if (st) return st;
  if (E < 1 || E > 65535) return fail(W8_E_INVALID, "E must be in [1, 65535]");
  if (T < 1) return fail(W8_E_INVALID, "T must be positive");
  return W8_OK;
}

w8_status resolve_moe(int fmt, int E, int T, int N, int K, int max_m, int packed, bool fused,
                      const w8_cfg* cfg, w8_cfg* out) {
  if (cfg) {
    w8_status st = check_moe_cfg(fmt, E, max_m, N, K, packed, *cfg, fused);
    if (st) return st;
    *out = *cfg;
  } else {
    *out = moe_default_cfg(fmt, E, T, max_m, N, K, packed, fused, nullptr);
    w8_status st = check_moe_cfg(fmt, E, max_m, N, K, packed, *out, fused);
    if (st) return st;
  }
  return W8_OK;
}

// Argument checks shared by w8_moe_gemm and w8_moe_linear (activations
// checked by the caller), then the launch.
w8_status moe_entry(MoeCall call, const w8_cfg* cfg, bool fused, w8_stream stream) {
  const int fmt = call.fmt, E = call.E, T = call.T, N = call.N, K = call.K, max_m = call.max_m;
  if (call.n_rows < 0) return fail(W8_E_INVALID, "n_rows must be >= 0");
  const bool empty = call.n_rows == 0;  // no routed entry: nothing to compute
  if (!call.offsets || !call.wq || !call.sw || (!empty && (!call.rows || !call.y)))
    return fail(W8_E_INVALID, "null device pointer");
  const int packed = call.ldw == 0;
  if (!aligned(call.wq, 16) || call.w_stride % 16)
    return fail(W8_E_INVALID, "wq and w_stride must be 16-byte aligned");
  if (packed) {
    if (call.w_stride < (long long)packed_weight_bytes(fmt, N, K, 1))
      return fail(W8_E_INVALID, "w_stride below one expert's packed weights");
  } else {
    if (call.ldw < K || call.ldw % 16)
      return fail(W8_E_INVALID, "ldw must be 0 (packed) or >= K, % 16");
    if (call.w_stride < (long long)N * call.ldw)
      return fail(W8_E_INVALID, "w_stride below N * ldw");
  }
  const long long nsw =
      fmt == W8_BLOCK_FP8 ? (long long)((N + 127) / 128) * (K / W8_GROUP) : (long long)N;
  if (call.sw_stride < nsw)
    return fail(W8_E_INVALID, "sw_stride below one expert's weight scales");
  if (call.ldy < N) return fail(W8_E_INVALID, "output leading dimension must be >= N");
  if (!aligned(call.sw, 4) || !aligned(call.y, 2) || !aligned(call.offsets, 4) ||
      !aligned(call.rows, 4))
    return fail(W8_E_INVALID, "misaligned scale, routing or output pointer");
  w8_cfg c;
  w8_status st = resolve_moe(fmt, E, T, N, K, max_m, packed, fused, cfg, &c);
  if (st) return st;
  const size_t need = moe_ws_bytes(fmt, E, T, max_m, N, K, c);
  if (need > 0 && !empty) {
    if (!call.ws || call.ws_bytes < need)
      return fail(W8_E_WORKSPACE, "workspace of " + std::to_string(need) + " bytes needed, got " +
                                      std::to_string(call.ws ? call.ws_bytes : 0));
    if (!aligned(call.ws, 16)) return fail(W8_E_INVALID, "workspace must be 16-byte aligned");
  }
  st = check_device();
  if (st) return st;
  if (!empty) {
    st = launch_moe_call(call, c, static_cast<hipStream_t>(stream));
    if (st) return st;
  }
  return ok();
}

}  // namespace

w8_status launch_moe_call(const MoeCall& g, const w8_cfg& c, hipStream_t s) {
  const int fmt = g.fmt, E = g.E, T = g.T, N = g.N, K = g.K, max_m = g.max_m;
  const int packed = g.ldw == 0;
  if (g.x && c.quant_launch) {
    // quantize the tokens into the workspace, then the kernel on the codes
    const MoeQuantWs w = moe_quant_ws(fmt, T, K, shared_ws_bytes(fmt, E, max_m, N, K, c));
    char* base = static_cast<char*>(g.ws);
    uint8_t* xq = reinterpret_cast<uint8_t*>(base + w.codes);
    float* sx = reinterpret_cast<float*>(base + w.scales);
    QuantActArgs q{static_cast<const uint16_t*>(g.x), xq, sx, g.ldx, w.ldq, T, K};
    hipError_t e = launch_quantize_act(fmt, q, s);
    if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("quantize_act launch", e));
    MoeCall gg = g;
    gg.x = nullptr;
    gg.ldx = 0;
    gg.xq = xq;
    gg.ldq = w.ldq;
    gg.sx = sx;
    gg.ws_bytes = w.codes;
    return launch_moe_call(gg, c, s);
  }
  const bool in_kernel = g.x != nullptr;
  const MoeLaunchFn fn = moe_fn(fmt, max_m, packed, c, in_kernel);
  if (!fn) return fail(W8_E_INVALID, "no compiled grouped kernel for this config");
  const bool shared = c.split_k > 1 || c.grid > 0;
  const int ntiles = tiles_of(N, c);
  GemmArgs a;
  std::memset(&a, 0, sizeof a);
  // in_kernel: the kernel reads bf16 activations (row stride in elements)
  a.xq = static_cast<const uint8_t*>(in_kernel ? g.x : g.xq);
  a.sx = in_kernel ? nullptr : g.sx;
  a.wq = static_cast<const uint8_t*>(g.wq);
  a.sw = g.sw;
  a.out = g.y;
  a.ldq = in_kernel ? g.ldx : g.ldq;
  a.ldw = g.ldw;
  a.ldo = g.ldy;
  a.M = max_m;  // per expert: its routed count (at most max_m rows are computed)
  a.N = N;
  a.K = K;
  a.ksteps = ksteps_of(fmt, K);
  a.kfull = K / kstep_of(fmt);
  a.split_k = c.split_k;
  a.split_shift = __builtin_ctz((unsigned)c.split_k);
  a.grid = c.grid;
  a.slots = partial_slots(fmt, N, K, c);
  a.ntiles = ntiles;
  a.sgroups = fmt == W8_BLOCK_FP8 ? K / W8_GROUP : 0;
  a.out_mode = 0;
  MoeArgs m;
  m.offsets = g.offsets;
  m.rows = g.rows;
  m.w_stride = g.w_stride;
  m.sw_stride = g.sw_stride;
  m.part_stride = (long long)part_stride(fmt, max_m, N, K, c);
  m.xrow_max = T - 1;
  m.n_rows = g.n_rows;
  m.n_experts = E;
  // With ascending offsets at most n_rows experts have entries: below E, a
  // grid of n_rows expert slots replaces one of E experts that mostly exit.
  m.compact = E <= kMoeCompactMaxE && g.n_rows > 0 && g.n_rows < E;
  const unsigned gy = m.compact ? (unsigned)g.n_rows : (unsigned)E;
  if (shared) {
    a.counters = static_cast<unsigned int*>(g.ws);
    a.part = static_cast<char*>(g.ws) + ws_counter_bytes(ntiles);
  }
  const unsigned wgs = c.grid > 0 ? (unsigned)c.grid : (unsigned)(ntiles * c.split_k);
  hipError_t e = fn(a, m, dim3(wgs, gy), dim3(64 * c.waves_k * c.waves_n), s);
  if (e != hipSuccess) return fail(W8_E_HIP, hip_msg("MoE GEMM launch", e));
  return W8_OK;
}

}  // namespace w8

using namespace w8;

extern "C" w8_status w8_moe_config(w8_fmt fmt_in, int E, int T, int N, int K, int max_m, int packed,
                                   w8_cfg* out, int* from_table) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_moe_shape(fmt, E, T, N, K, max_m);
  if (st) return st;
  if (!out) return fail(W8_E_INVALID, "null output pointer");
  *out = moe_default_cfg(fmt, E, T, max_m, N, K, packed ? 1 : 0, false, from_table);
  return ok();
}

extern "C" w8_status w8_moe_linear_config(w8_fmt fmt_in, int E, int T, int N, int K, int max_m,
                                          int packed, w8_cfg* out, int* from_table) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_moe_shape(fmt, E, T, N, K, max_m);
  if (st) return st;
  if (!out) return fail(W8_E_INVALID, "null output pointer");
  *out = moe_default_cfg(fmt, E, T, max_m, N, K, packed ? 1 : 0, true, from_table);
  return ok();
}

extern "C" w8_status w8_moe_validate_config(w8_fmt fmt_in, int E, int N, int K, int max_m,
                                            int packed, const w8_cfg* cfg) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_moe_shape(fmt, E, 1, N, K, max_m);
  if (st) return st;
  if (!cfg) return fail(W8_E_INVALID, "null cfg");
  st = check_moe_cfg(fmt, E, max_m, N, K, packed ? 1 : 0, *cfg, false);
  if (st) return st;
  return ok();
}

extern "C" w8_status w8_moe_workspace_size(w8_fmt fmt_in, int E, int T, int N, int K, int max_m,
                                           int packed, const w8_cfg* cfg, size_t* bytes) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_moe_shape(fmt, E, T, N, K, max_m);
  if (st) return st;
  if (!bytes) return fail(W8_E_INVALID, "null output pointer");
  w8_cfg c;
  if (cfg) {  // a config of either grouped op
    st = check_moe_cfg(fmt, E, max_m, N, K, packed ? 1 : 0, *cfg, false);
    if (st) st = check_moe_cfg(fmt, E, max_m, N, K, packed ? 1 : 0, *cfg, true);
    if (st) return st;
    c = *cfg;
  } else {
    st = resolve_moe(fmt, E, T, N, K, max_m, packed ? 1 : 0, false, nullptr, &c);
    if (st) return st;
  }
  *bytes = moe_ws_bytes(fmt, E, T, max_m, N, K, c);
  return ok();
}

extern "C" w8_status w8_moe_gemm(w8_fmt fmt_in, int E, int T, int N, int K, int max_m,
                                 const void* xq, int64_t ldq, const float* sx,
                                 const int32_t* offsets, const int32_t* rows, int n_rows,
                                 const void* wq, int64_t ldw, int64_t w_stride, const float* sw,
                                 int64_t sw_stride, void* y, int64_t ldy, const w8_cfg* cfg,
                                 void* ws, size_t ws_bytes, w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_moe_shape(fmt, E, T, N, K, max_m);
  if (st) return st;
  if (!xq || !sx) return fail(W8_E_INVALID, "null device pointer");
  if (!aligned(xq, 16) || ldq < K || ldq % 16)
    return fail(W8_E_INVALID, "xq must be 16-byte aligned with ldq >= K and ldq % 16 == 0");
  if (!aligned(sx, 4)) return fail(W8_E_INVALID, "misaligned scale, routing or output pointer");
  MoeCall call{fmt, E,  T,        N,  K,   max_m,   xq,  ldq, sx,       offsets, rows, n_rows,
               wq,  ldw, w_stride, sw, sw_stride, y, ldy, ws,  ws_bytes, nullptr, 0};
  return moe_entry(call, cfg, false, stream);
}

extern "C" w8_status w8_moe_linear(w8_fmt fmt_in, int E, int T, int N, int K, int max_m,
                                   const void* x, int64_t ldx, const int32_t* offsets,
                                   const int32_t* rows, int n_rows, const void* wq, int64_t ldw,
                                   int64_t w_stride, const float* sw, int64_t sw_stride, void* y,
                                   int64_t ldy, const w8_cfg* cfg, void* ws, size_t ws_bytes,
                                   w8_stream stream) {
  const int fmt = raw_enum(fmt_in);
  w8_status st = check_moe_shape(fmt, E, T, N, K, max_m);
  if (st) return st;
  if (!x) return fail(W8_E_INVALID, "null device pointer");
  if (!aligned(x, 16) || ldx % 8 || ldx < K)
    return fail(W8_E_INVALID, "x must be 16-byte aligned with ldx >= K and ldx % 8 == 0");
  MoeCall call{fmt, E,  T,        N,  K,   max_m,   nullptr, 0,   nullptr,  offsets, rows, n_rows,
               wq,  ldw, w_stride, sw, sw_stride, y,       ldy, ws,       ws_bytes, x,    ldx};
  return moe_entry(call, cfg, true, stream);
}
