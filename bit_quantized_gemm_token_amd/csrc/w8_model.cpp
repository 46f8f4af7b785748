// The config family's feasible set and a cost model that ranks it
// (flashinfer-ai/flashinfer pull 3948: a heuristic scores every feasible
// tactic to give a top-1 pick without tuning, and the autotuner profiles only
// the top-N of that ranking instead of the whole list; the pick is computed
// per M bucket, floor(log2 M)).
//
// The model predicts the time of one call from the quantities that bound
// this kernel on MI355X, with constants fitted to the tuner's measured
// timings (fit_model.py beside this package fits them through
// w8_predict_us, so the fit and the library evaluate one model):
//   - a fixed cost per launch (graph-replayed kernel start and drain);
//   - the busiest compute unit's bytes through its vector memory path, at a
//     rate set by Little's law -- the bytes its resident waves keep in
//     flight (two stages of U K-steps of weight and activation fragments)
//     over the load latency -- capped by the per-CU path's peak;
//   - the whole call's weight bytes at the HBM rate;
//   - per workgroup on the busiest CU, a start-up cost and its MFMA time;
//     the LDS reduction of its K-waves;
//   - the split-K or stream-K reduction chain, the fused quantization's
//     staging (and, per token, its whole-row pass), or the separate
//     quantize launch.
// The busiest CU's time and the HBM time overlap; the rest add.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <mutex>
#include <tuple>
#include <vector>

#include "w8_internal.hpp"

namespace w8 {

namespace {

// Fitted constants (us, bytes/us), in this order in w8_predict_us's
// params.  fit_model.py prints these from a dump of measured candidate
// timings.
struct ModelParams {
  double t0;          // fixed cost per launch
  double cu_bw;       // per-CU vector-memory peak
  double latency;     // load latency under load
  double hbm_bw;      // sustained HBM read rate of the weights
  double slots;       // workgroups resident per CU
  double sk_base;     // shared-tile reduction chain, fixed part
  double sk_slot;     // per partial slot read by the last arriver
  double xl_stage;    // x_lds staging: copy, wait and barrier
  double wg_cost;     // per workgroup a CU runs (start, prologue, epilogue)
  double mfma;        // per MFMA K-step of a workgroup, per SIMD it spreads over
  double reduce;      // per extra K-wave and output block reduced through LDS
  double q_launch;    // a separate quantize launch
  double q_row_bw;    // per-CU rate of the fused per-token whole-row pass
};

constexpr ModelParams kParams = {1.6537, 56705.2, 1.0003, 4.54169e6, 2.608, 1.2018, 1.5197,
                                 0.43, 0.1419, 0.0146, 0.051, 0.225973, 20816.5};
constexpr int kParamCount = (int)(sizeof(ModelParams) / sizeof(double));
static_assert(kParamCount == 13, "w8_predict_us documents 13 constants");

int kstep_bytes(int fmt) { return fmt == W8_W8A8_INT8 ? 64 : 128; }

double predict_with(const ModelParams& p, int fmt, int op, int M, int N, int K, const w8_cfg& c,
                    int layout) {
  // The K-segmented layouts fit the same terms: a K-loop step is a span of
  // layout K-steps, a block R = 16/layout weight rows (still one fragment of
  // 16 x K-step bytes per load), and M runs as launches of at most 2R rows.
  const int R = layout_rows(layout);
  const int launches = (M + 2 * R - 1) / (2 * R);
  if (launches > 1) {
    const int rows = 2 * R, last = M - (launches - 1) * rows;
    return (launches - 1) * predict_with(p, fmt, op, rows, N, K, c, layout) +
           predict_with(p, fmt, op, last, N, K, c, layout);
  }
  const int T = layout_spans(fmt, K, layout);
  const double KS = kstep_bytes(fmt);
  const int MB = (M + R - 1) / R, NB = c.tile_n / R, W = c.waves_k * c.waves_n;
  const long long ntiles = tiles_of(N, c);
  const long long G = c.grid > 0 ? c.grid : ntiles * c.split_k;
  const double seg = c.grid > 0 ? std::ceil((double)ntiles * T / c.grid)
                                : std::ceil((double)T / c.split_k);
  const bool fused = op == W8_OP_LINEAR && !c.quant_launch;
  // bytes one workgroup moves through its CU's vector memory path
  const double wbytes = 16.0 * NB * c.waves_n * seg * KS;
  double abytes = (c.x_lds ? 1.0 : (double)c.waves_n) * 16.0 * MB * seg * KS;
  if (fused) abytes *= 2.0;  // bf16 activations
  const bool shared = c.split_k > 1 || c.grid > 0;
  const double pbytes = shared ? 16.0 * NB * c.waves_n * 16.0 * MB * 4.0 : 0.0;
  const double per_wg = wbytes + abytes + pbytes;
  // work rounds on the busiest CU and the bytes its resident waves keep in flight
  const double per_cu_wgs = std::ceil((double)G / 256.0);
  const double resident = std::min(per_cu_wgs, p.slots);
  const double frag = 64.0 * 16.0 * (KS / 64.0);  // one fragment load of a wave
  const double inflight =
      resident * W * 2.0 * c.unroll * (NB + (c.x_lds ? 0.0 : MB)) * frag;
  const double rate = std::min(p.cu_bw, inflight / p.latency);
  const double t_cu = per_cu_wgs * per_wg / rate;
  const double t_hbm = (double)N * K / p.hbm_bw;
  double t = p.t0 + std::max(t_cu, t_hbm);
  t += per_cu_wgs * p.wg_cost;
  t += p.mfma * per_cu_wgs * seg * NB * MB * (KS / 64.0) / std::max(1, std::min(W, 4));
  t += p.reduce * (c.waves_k - 1) * NB * MB;
  if (shared) {
    const int slots = partial_slots(fmt, N, K, c);
    t += p.sk_base + p.sk_slot * slots * 16.0 * NB * c.waves_n * 16.0 * MB * 4.0 / p.cu_bw;
  }
  if (c.x_lds) t += p.xl_stage;
  if (fused && fmt != W8_BLOCK_FP8) t += 2.0 * M * K / p.q_row_bw;
  if (op == W8_OP_LINEAR && c.quant_launch) t += p.q_launch;
  return t;
}

}  // namespace

double predict_us(int fmt, int op, int M, int N, int K, const w8_cfg& c, int layout) {
  return predict_with(kParams, fmt, op, M, N, K, c, layout);
}

std::vector<w8_cfg> enumerate_configs(int fmt, int op, int M, int N, int K, int layout,
                                      int max_split_k, int stream_k, bool prune_waves) {
  const int T = layout_spans(fmt, K, layout);
  const int R = layout_rows(layout);
  const long long wbytes = (long long)N * ((K + 15) / 16 * 16);
  const int tiles_n[] = {R, 2 * R, 4 * R};
  // (waves_k, waves_n, x_lds)
  const int wave_shapes[][3] = {{1, 1, 0}, {2, 1, 0}, {4, 1, 0}, {8, 1, 0}, {16, 1, 0},
                                {1, 1, 1}, {2, 1, 1}, {4, 1, 1}, {8, 1, 1},
                                {1, 2, 1}, {1, 4, 1}, {1, 8, 1}};
  const int unrolls[] = {1, 2, 4};
  const int grids[] = {256, 512, 1024};
  auto total_waves = [&](const w8_cfg& c) {
    const long long wgs = c.grid > 0 ? c.grid : (long long)tiles_of(N, c) * c.split_k;
    return wgs * c.waves_k * c.waves_n;
  };
  std::vector<w8_cfg> all;
  long long most_waves = 0;
  auto consider = [&](const w8_cfg& c) {
    if (check_cfg(fmt, op, M, N, K, c, layout) != W8_OK) return;
    const long long per_wave = c.grid > 0 ? (long long)tiles_of(N, c) * T / (c.grid * c.waves_k)
                                          : (long long)T / (c.split_k * c.waves_k);
    if (per_wave < 1) return;
    if (c.unroll > 1 && per_wave < c.unroll) return;
    if ((long long)workspace_bytes(fmt, op, M, N, K, c, layout) >
        2 * wbytes + (long long)ws_counter_bytes(0))
      return;
    all.push_back(c);
    most_waves = std::max(most_waves, total_waves(c));
  };
  for (int tn : tiles_n)
    for (const auto& ws : wave_shapes)
      for (int u : unrolls)
        for (int sw = 0; sw < 2; ++sw) {
          w8_cfg c;
          std::memset(&c, 0, sizeof c);
          c.abi_version = W8_ABI_VERSION;
          c.tile_n = tn;
          c.waves_k = ws[0];
          c.waves_n = ws[1];
          c.x_lds = ws[2];
          c.unroll = u;
          c.swap_ab = sw;
          for (int s = 1; s <= max_split_k; s *= 2) {
            c.split_k = s;
            c.grid = 0;
            consider(c);
          }
          for (int gr : grids) {
            if (!stream_k) break;
            c.split_k = 1;
            c.grid = gr;
            consider(c);
          }
        }
  const long long min_waves = prune_waves ? std::min<long long>(256, most_waves) : 0;
  std::vector<w8_cfg> out;
  for (const w8_cfg& c : all)
    if (total_waves(c) >= min_waves) out.push_back(c);
  // The linear op also competes with a quantize launch of its own followed
  // by the GEMM: with the GEMM's config for this shape and layout (its table
  // entry when the GEMM was tuned first) and with the GEMM's default.
  if (op == W8_OP_LINEAR) {
    int hit = 0;
    std::vector<w8_cfg> gemm_cfgs = {resolve_cfg(fmt, W8_OP_GEMM, M, N, K, layout, &hit)};
    gemm_cfgs.push_back(make_default_cfg(fmt, W8_OP_GEMM, M, N, K, layout));
    for (w8_cfg c : gemm_cfgs) {
      c.quant_launch = 1;
      if (check_cfg(fmt, op, M, N, K, c, layout) != W8_OK) continue;
      bool dup = false;
      for (const w8_cfg& e : out) dup = dup || std::memcmp(&e, &c, sizeof c) == 0;
      if (!dup) out.push_back(c);
    }
  }
  return out;
}

std::vector<std::pair<double, w8_cfg>> rank_configs(int fmt, int op, int M, int N, int K,
                                                    int layout, int max_split_k, int stream_k) {
  std::vector<std::pair<double, w8_cfg>> r;
  for (const w8_cfg& c : enumerate_configs(fmt, op, M, N, K, layout, max_split_k, stream_k))
    r.emplace_back(predict_us(fmt, op, M, N, K, c, layout), c);
  // stable: equal predictions keep enumeration order
  std::stable_sort(r.begin(), r.end(),
                   [](const auto& a, const auto& b) { return a.first < b.first; });
  return r;
}

// The GEMM's picks are memoized per shape (they depend on nothing else); the
// linear op's depend on the table's GEMM entry, so they are recomputed.
w8_cfg model_cfg(int fmt, int op, int M, int N, int K, int layout) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int>, w8_cfg> memo;
  const auto key = std::make_tuple(fmt, layout, M, N, K);
  if (op == W8_OP_GEMM) {
    std::lock_guard<std::mutex> lk(mu);
    auto it = memo.find(key);
    if (it != memo.end()) return it->second;
  }
  const auto r = rank_configs(fmt, op, M, N, K, layout, W8_MAX_SPLIT_K, 0);
  const w8_cfg c = r.empty() ? make_default_cfg(fmt, op, M, N, K, layout) : r.front().second;
  if (op == W8_OP_GEMM) {
    std::lock_guard<std::mutex> lk(mu);
    memo[key] = c;
  }
  return c;
}

}  // namespace w8

extern "C" w8_status w8_predict_us(int n, const int* fmt, const int* op, const int* layout,
                                   const int* M, const int* N, const int* K, const w8_cfg* cfgs,
                                   const double* params, int nparams, double* us) {
  if (n < 0 || (n > 0 && (!fmt || !op || !layout || !M || !N || !K || !cfgs || !us)))
    return w8::fail(W8_E_INVALID, "bad arguments");
  w8::ModelParams p = w8::kParams;
  if (params) {
    if (nparams != w8::kParamCount)
      return w8::fail(W8_E_INVALID, "params must hold the model's 13 constants");
    std::memcpy(&p, params, sizeof p);
  }
  for (int i = 0; i < n; ++i) {
    const w8_cfg& c = cfgs[i];
    // what the arithmetic divides by or indexes with
    if (fmt[i] < 0 || fmt[i] > 2 || M[i] < 1 || N[i] < 1 || K[i] < 1 ||
        !w8::layout_valid(layout[i]) || c.tile_n < 1 || c.waves_k < 1 || c.waves_n < 1 ||
        c.unroll < 1 || c.split_k < 1 || c.grid < 0)
      return w8::fail(W8_E_INVALID, "row " + std::to_string(i) + ": bad shape, layout or config");
    us[i] = w8::predict_with(p, fmt[i], op[i], M[i], N[i], K[i], c, layout[i]);
  }
  return w8::ok();
}

extern "C" w8_status w8_model_config(w8_fmt fmt_in, w8_op op_in, int M, int N, int K, int layout,
                                     w8_cfg* out) {
  const int fmt = w8::raw_enum(fmt_in);
  const int op = w8::raw_enum(op_in);
  w8_status st = w8::check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!out) return w8::fail(W8_E_INVALID, "null output pointer");
  if (op != W8_OP_GEMM && op != W8_OP_LINEAR) return w8::fail(W8_E_INVALID, "unknown op");
  if (!w8::layout_valid(layout))
    return w8::fail(W8_E_INVALID, "weight layout must be 0, 1, 2, 4 or 8");
  *out = w8::model_cfg(fmt, op, M, N, K, layout);
  return w8::ok();
}
