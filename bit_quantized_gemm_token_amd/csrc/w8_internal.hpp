// Host-side internals shared by the C-ABI, the config table and the tuner.
#pragma once
#include <hip/hip_runtime.h>

#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "../../include/w8gemm.h"
#include "w8_launch.hpp"

namespace w8 {

// The integer a C caller passed for an enum-typed argument.  The C-ABI's
// enums have no fixed underlying type, so in C++ a value outside their range
// may not be loaded as the enum; the entry points copy the argument's bytes
// into an int and validate that instead.
// (By reference: passing the argument by value would load it as the enum.)
template <class E>
inline int raw_enum(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

// Thread-local error text behind w8_last_error().
w8_status fail(w8_status s, const std::string& msg);
w8_status ok();
std::string hip_msg(const char* what, hipError_t e);

const char* fmt_name(int fmt);
int fmt_from_name(const std::string& s);  // -1 if unknown

// Shape checks shared by the GEMM, the quantizer and the tuner.
w8_status check_gemm_shape(int fmt, int M, int N, int K);
// Config checks (shape-independent and shape-dependent) for operation op on
// weights of layout `layout` (0 row-major; 1, 2, 4, 8 packed with that many
// K-steps per MFMA).
w8_status check_cfg(int fmt, int op, int M, int N, int K, const w8_cfg& c, int layout);
w8_cfg make_default_cfg(int fmt, int op, int M, int N, int K, int layout);
size_t workspace_bytes(int fmt, int op, int M, int N, int K, const w8_cfg& c, int layout);
// The layout of a GEMM call's ldw (-1 if invalid): > 0 row-major, 0 (or -1)
// plain packed, -2/-4/-8 K-segmented packed.
int layout_from_ldw(long long ldw);
// Workspace regions of the linear op with quant_launch == 1 (byte offsets):
// the GEMM's part at 0, the activation codes (row stride ldq) and scales.
struct LinearWs {
  size_t codes, scales, total;
  long long ldq;
};
LinearWs linear_ws(int fmt, int M, int N, int K, const w8_cfg& c, int layout);
int tiles_of(int N, const w8_cfg& c);                       // output tiles along N
int partial_slots(int fmt, int N, int K, const w8_cfg& c);  // workspace slots per tile
int ksteps_of(int fmt, int K);

// Resolve cfg == NULL: the table entry for the shape (*from_table = 1), else
// one for the same N, K and an M of the same floor(log2 M) bucket that is
// valid for this M (2), else the cost model's pick (0).
w8_cfg resolve_cfg(int fmt, int op, int M, int N, int K, int layout, int* from_table);

// The config family's feasible set for the tuner (its pruning rules, and for
// the linear op the quantize-launch variants), the cost model's predicted
// time per call of a config, the set ranked by it (ascending), and the
// model's top-1 pick.
std::vector<w8_cfg> enumerate_configs(int fmt, int op, int M, int N, int K, int layout,
                                      int max_split_k, int stream_k, bool prune_waves = true);
double predict_us(int fmt, int op, int M, int N, int K, const w8_cfg& c, int layout);
std::vector<std::pair<double, w8_cfg>> rank_configs(int fmt, int op, int M, int N, int K,
                                                    int layout, int max_split_k, int stream_k);
w8_cfg model_cfg(int fmt, int op, int M, int N, int K, int layout);

// The device must be gfx950 (checked once per device).
w8_status check_device();

// Launch one GEMM (arguments already validated).
struct GemmCall {
  int fmt, M, N, K;
  const void* xq;
  long long ldq;
  const float* sx;
  const void* wq;
  long long ldw;
  const float* sw;
  void* out;
  long long ldo;
  int out_mode;
  void* ws;
  size_t ws_bytes;
  int layout;         // weight layout: 0 row-major, 1/2/4/8 packed
  const void* x;      // fused quantization (w8_linear): bf16 activations, else null
  long long ldx;
};
w8_status launch_gemm_call(const GemmCall& call, const w8_cfg& c, hipStream_t s);
// The linear op (call.x set): the fused GEMM, or with c.quant_launch the
// quantize kernel into the workspace and then the GEMM.
w8_status launch_linear_call(const GemmCall& call, const w8_cfg& c, hipStream_t s);

// MoE grouped GEMM (w8_moe.cpp).
struct MoeCall {
  int fmt, E, T, N, K, max_m;
  const void* xq;
  long long ldq;
  const float* sx;
  const int* offsets;
  const int* rows;
  int n_rows;
  const void* wq;
  long long ldw;  // 0: packed
  long long w_stride;
  const float* sw;
  long long sw_stride;
  void* y;
  long long ldy;
  void* ws;
  size_t ws_bytes;
  const void* x;  // non-null: bf16 activations, quantization fused (xq, sx unused)
  long long ldx;  // elements
};
// fused: the rules of the fused grouped kernel (w8_moe_linear).
w8_status check_moe_cfg(int fmt, int E, int max_m, int N, int K, int packed, const w8_cfg& c,
                        bool fused);
size_t moe_ws_bytes(int fmt, int E, int T, int max_m, int N, int K, const w8_cfg& c);
w8_cfg moe_fallback_cfg(int fmt, int E, int T, int max_m, int N, int K, int packed, bool fused);
w8_status launch_moe_call(const MoeCall& call, const w8_cfg& c, hipStream_t s);

constexpr const char* kArch = "gfx950";

}  // namespace w8
