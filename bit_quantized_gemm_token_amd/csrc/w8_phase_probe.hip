// Phase probe: where the time of one GEMM launch goes.
//
// A timing study, not part of the library: it compiles the GEMM kernel with
// the phase stamps switched on (W8_PHASE_STAMPS, see w8_gemm.hpp) for a
// fixed list of configurations -- the kinds of kernel the tuned table picks
// on the benchmark sweep -- and replays each from a HIP graph the way the
// benchmark does (R launches on R rotating weight copies spanning >= 1 GiB).
// The per-launch time comes from HIP events around the graph; the phases
// come from the stamps of one more replay: for each launch, the gap since
// the previous launch's last workgroup finished, the spread of workgroup
// start times, and per workgroup the K loop (wave 0 and the slowest wave),
// the K-wave sum, and for shared tiles the partials' acknowledgement, the
// arrival count and the last arriver's partial reads + epilogue; for owned
// tiles the epilogue.  Inputs are random codes (no E4M3FN NaN) and constant
// scales: the arithmetic does not matter here, only the memory traffic and
// the control path, which are those of the benchmark's calls.
//
// Output: one JSON object per configuration on stdout.  Usage:
//   w8_phase_probe [substring]   (only the configurations whose name has it)
#define W8_PHASE_STAMPS (1 << 20)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "w8_gemm.hpp"

using namespace w8;

namespace {

#define CK(x)                                                                         \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                   \
    }                                                                                 \
  } while (0)

struct Cfg {
  const char* name;
  int fmt, M, N, K;
  int T;  // weight layout: 0 row-major, 1 packed, 2/4/8 K-segmented
  int MB, NB, WK, WN, U, SWAP, XL, split;
  GemmLaunchFn fn;
};

#define W8_PROBE(name, F, M, N, K, T, MB, NB, WK, WN, U, SW, XL, SPLIT)          \
  {name, F, M, N, K, T, MB, NB, WK, WN, U, SW, XL, SPLIT,                         \
   &launch_gemm<F, MB, NB, WK, WN, U, SW, T, XL, 0>}

// (name, fmt, M, N, K, layout, MB, NB, WK, WN, unroll, swap_ab, x_lds, split_k):
// configurations of the kinds the shipped table picks on the sweep.
const Cfg kCfgs[] = {
    W8_PROBE("FP8 1x512x7168 seg8", 0, 1, 512, 7168, 8, 1, 1, 1, 1, 4, 0, 0, 1),
    W8_PROBE("FP8 1x896x1024 seg8", 0, 1, 896, 1024, 8, 1, 1, 1, 1, 1, 0, 0, 1),
    W8_PROBE("FP8 1x5120x8192 seg4", 0, 1, 5120, 8192, 4, 1, 1, 1, 1, 4, 0, 0, 1),
    W8_PROBE("FP8 8x896x5120 seg4 k8", 0, 8, 896, 5120, 4, 2, 1, 8, 1, 1, 0, 0, 1),
    W8_PROBE("W8A8 8x5120x8192 seg2 k2", 1, 8, 5120, 8192, 2, 1, 1, 2, 1, 2, 0, 0, 1),
    W8_PROBE("FP8 8x3584x5120 packed k8", 0, 8, 3584, 5120, 1, 1, 1, 8, 1, 1, 0, 0, 1),
    W8_PROBE("Block 8x3584x5120 packed k8", 2, 8, 3584, 5120, 1, 1, 1, 8, 1, 1, 0, 0, 1),
    W8_PROBE("FP8 16x512x7168 packed s8", 0, 16, 512, 7168, 1, 1, 1, 1, 1, 4, 0, 0, 8),
    W8_PROBE("FP8 32x512x7168 packed s8", 0, 32, 512, 7168, 1, 2, 1, 1, 1, 4, 0, 0, 8),
    W8_PROBE("FP8 32x896x1024 packed k8 xlds", 0, 32, 896, 1024, 1, 2, 1, 8, 1, 1, 0, 1, 1),
    W8_PROBE("FP8 16x4608x7168 packed s8", 0, 16, 4608, 7168, 1, 1, 1, 1, 1, 1, 0, 0, 8),
    W8_PROBE("FP8 32x4608x7168 packed n8 s4 xlds", 0, 32, 4608, 7168, 1, 2, 1, 1, 8, 1, 0, 1, 4),
};

constexpr long long kOutBytes = 2LL << 20;  // per launch: Y in the first MiB, stamps after
constexpr long long kRotate = 1LL << 30;

template <int KSTEP, int T>
void pack(const uint8_t* w, int N, int K, int spans, uint8_t* out, long long bytes,
          hipStream_t s) {
  const long long chunks = bytes / 16;
  hipLaunchKernelGGL((pack_weight_kernel<KSTEP, T>), dim3((unsigned)((chunks + 255) / 256)),
                     dim3(256), 0, s, w, (long long)K, N, K, spans, out, chunks);
  CK(hipGetLastError());
}

void pack_any(int kstep, int T, const uint8_t* w, int N, int K, int spans, uint8_t* out,
              long long bytes, hipStream_t s) {
  if (kstep == 64) {
    if (T == 1) pack<64, 1>(w, N, K, spans, out, bytes, s);
    if (T == 2) pack<64, 2>(w, N, K, spans, out, bytes, s);
    if (T == 4) pack<64, 4>(w, N, K, spans, out, bytes, s);
    if (T == 8) pack<64, 8>(w, N, K, spans, out, bytes, s);
  } else {
    if (T == 1) pack<128, 1>(w, N, K, spans, out, bytes, s);
    if (T == 2) pack<128, 2>(w, N, K, spans, out, bytes, s);
    if (T == 4) pack<128, 4>(w, N, K, spans, out, bytes, s);
    if (T == 8) pack<128, 8>(w, N, K, spans, out, bytes, s);
  }
}

struct Stat {
  double sum = 0, mx = 0;
  long long n = 0;
  void add(double v) {
    sum += v;
    n++;
    mx = std::max(mx, v);
  }
  double avg() const { return n ? sum / n : 0.0; }
};

void run(const Cfg& c, hipStream_t s) {
  const int kstep = c.fmt == 1 ? 64 : 128;
  const int T = c.T > 1 ? c.T : 1;
  const int R = 16 / T;
  const int spans = ((c.K + kstep - 1) / kstep + T - 1) / T;
  const long long wbytes =
      c.T ? (long long)((c.N + R - 1) / R) * spans * 16 * kstep : (long long)c.N * c.K;
  const long long copies = std::min<long long>(1000, (kRotate + wbytes - 1) / wbytes);
  const int ntiles = (c.N + R * c.NB * c.WN - 1) / (R * c.NB * c.WN);
  const int wgs = ntiles * c.split;
  const int nw = c.WK * c.WN;
  // the kernel's assumptions: rows of one launch, x_lds capacity, record size
  if (c.M > R * c.MB || (long long)c.M * c.N * 2 > W8_PHASE_STAMPS ||
      (long long)wgs * 256 > kOutBytes - W8_PHASE_STAMPS || nw > 24 ||
      (c.XL && (spans / c.split) * c.MB * (kstep / 64) > kXlChunks)) {
    std::fprintf(stderr, "%s: configuration outside the probe's limits\n", c.name);
    std::exit(1);
  }
  std::vector<uint8_t> h((size_t)c.N * c.K);
  unsigned st = 12345u;
  for (auto& b : h) {
    st = st * 1664525u + 1013904223u;
    b = (uint8_t)((st >> 24) & 0x77);  // finite codes in both formats
  }
  uint8_t *wrow, *pool, *xq;
  CK(hipMalloc(&wrow, h.size()));
  CK(hipMemcpy(wrow, h.data(), h.size(), hipMemcpyHostToDevice));
  CK(hipMalloc(&pool, copies * wbytes));
  for (long long r = 0; r < copies; ++r) {
    if (c.T)
      pack_any(kstep, T, wrow, c.N, c.K, spans, pool + r * wbytes, wbytes, s);
    else
      CK(hipMemcpyAsync(pool + r * wbytes, wrow, wbytes, hipMemcpyDeviceToDevice, s));
  }
  std::vector<uint8_t> hx((size_t)c.M * c.K);
  for (auto& b : hx) {
    st = st * 1664525u + 1013904223u;
    b = (uint8_t)((st >> 24) & 0x77);
  }
  CK(hipMalloc(&xq, hx.size()));
  CK(hipMemcpy(xq, hx.data(), hx.size(), hipMemcpyHostToDevice));
  const int groups = c.K / 128;
  const size_t nsx = c.fmt == 2 ? (size_t)c.M * groups : c.M;
  const size_t nsw = c.fmt == 2 ? (size_t)((c.N + 127) / 128) * groups : c.N;
  std::vector<float> hs(std::max(nsx, nsw), 0.01f);
  float *sx, *sw;
  CK(hipMalloc(&sx, nsx * 4));
  CK(hipMalloc(&sw, nsw * 4));
  CK(hipMemcpy(sx, hs.data(), nsx * 4, hipMemcpyHostToDevice));
  CK(hipMemcpy(sw, hs.data(), nsw * 4, hipMemcpyHostToDevice));
  char* outs;
  CK(hipMalloc(&outs, copies * kOutBytes));
  CK(hipMemset(outs, 0, copies * kOutBytes));
  const size_t cb = (size_t)kSplitKMaxTiles * kCounterWords * 4;
  const size_t pb = (size_t)ntiles * c.split * c.WN * c.NB * c.MB * 1024;
  char* ws;
  CK(hipMalloc(&ws, cb + pb + 256));
  CK(hipMemset(ws, 0, cb + pb + 256));
  CK(hipStreamSynchronize(s));

  auto args = [&](long long r) {
    GemmArgs a;
    a.xq = xq;
    a.sx = sx;
    a.wq = pool + r * wbytes;
    a.sw = sw;
    a.out = outs + r * kOutBytes;
    a.part = c.split > 1 ? ws + cb : nullptr;
    a.counters = c.split > 1 ? reinterpret_cast<unsigned*>(ws) : nullptr;
    a.ldq = c.K;
    a.ldw = c.T ? 0 : c.K;
    a.ldo = c.N;
    a.M = c.M;
    a.N = c.N;
    a.K = c.K;
    a.ksteps = spans;
    a.kfull = c.K / kstep / T;
    a.split_k = c.split;
    a.split_shift = __builtin_ctz((unsigned)c.split);
    a.grid = 0;
    a.slots = c.split;
    a.ntiles = ntiles;
    a.sgroups = c.fmt == 2 ? groups : 0;
    a.out_mode = 0;
    return a;
  };
  hipGraph_t g;
  hipGraphExec_t ge;
  CK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
  for (long long r = 0; r < copies; ++r)
    CK(c.fn(args(r), dim3((unsigned)wgs), dim3(64 * nw), s));
  CK(hipStreamEndCapture(s, &g));
  CK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  std::vector<float> ts;
  for (int i = 0; i < 9; ++i) {
    CK(hipEventRecord(e0, s));
    CK(hipGraphLaunch(ge, s));
    CK(hipEventRecord(e1, s));
    CK(hipEventSynchronize(e1));
    float ms;
    CK(hipEventElapsedTime(&ms, e0, e1));
    if (i >= 2) ts.push_back(ms * 1000.0f / (float)copies);
  }
  std::sort(ts.begin(), ts.end());
  // one more replay with cleared records, read back
  for (long long r = 0; r < copies; ++r)
    CK(hipMemsetAsync(outs + r * kOutBytes + W8_PHASE_STAMPS, 0, (size_t)wgs * 256, s));
  CK(hipGraphLaunch(ge, s));
  CK(hipStreamSynchronize(s));
  std::vector<unsigned long long> rec((size_t)copies * wgs * 32);
  for (long long r = 0; r < copies; ++r)
    CK(hipMemcpy(rec.data() + (size_t)r * wgs * 32, outs + r * kOutBytes + W8_PHASE_STAMPS,
                 (size_t)wgs * 256, hipMemcpyDeviceToHost));

  Stat gap, spread, busy, loop0, loopmax, ksum, ack, cnt, last, ep;
  unsigned long long prev_end = 0;
  for (long long r = 1; r < copies; ++r) {  // launch 0 follows no launch of this graph
    unsigned long long t0 = ~0ull, tstart_last = 0, t1 = 0;
    for (int w = 0; w < wgs; ++w) {
      const unsigned long long* q = &rec[((size_t)r * wgs + w) * 32];
      const unsigned long long end = std::max(q[6], q[7]);
      t0 = std::min(t0, q[0]);
      tstart_last = std::max(tstart_last, q[0]);
      t1 = std::max(t1, end);
      unsigned long long lm = 0;
      for (int v = 0; v < nw; ++v) lm = std::max(lm, q[8 + v]);
      loop0.add((double)q[1] - (double)q[0]);
      loopmax.add((double)lm - (double)q[0]);
      ksum.add((double)q[2] - (double)lm);
      if (c.split > 1) {
        ack.add((double)q[3] - (double)q[2]);
        cnt.add((double)q[4] - (double)q[3]);
        if (q[6]) last.add((double)q[6] - (double)q[4]);
      } else {
        ep.add((double)q[6] - (double)q[2]);
      }
    }
    busy.add((double)t1 - (double)t0);
    spread.add((double)tstart_last - (double)t0);
    if (prev_end) gap.add((double)t0 - (double)prev_end);
    prev_end = t1;
  }
  auto us = [](double ticks) { return ticks * 0.01; };  // 100 MHz
  std::printf(
      "{\"name\": \"%s\", \"grid\": %d, \"block\": %d, \"waves_k\": %d, \"launches\": %lld, "
      "\"us_per_launch\": %.3f, \"gap_us\": %.3f, \"in_kernel_us\": %.3f, "
      "\"start_spread_us\": %.3f, \"loop_wave0_us\": %.3f, \"loop_slowest_wave_us\": %.3f, "
      "\"kwave_sum_us\": %.3f, \"ack_us\": %.3f, \"count_us\": %.3f, "
      "\"last_arriver_us\": %.3f, \"epilogue_us\": %.3f}\n",
      c.name, wgs, 64 * nw, c.WK, copies, ts[ts.size() / 2], us(gap.avg()), us(busy.avg()),
      us(spread.avg()), us(loop0.avg()), us(loopmax.avg()), us(ksum.avg()), us(ack.avg()),
      us(cnt.avg()), us(last.avg()), us(ep.avg()));
  std::fflush(stdout);
  CK(hipGraphExecDestroy(ge));
  CK(hipGraphDestroy(g));
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  CK(hipFree(wrow));
  CK(hipFree(pool));
  CK(hipFree(xq));
  CK(hipFree(sx));
  CK(hipFree(sw));
  CK(hipFree(outs));
  CK(hipFree(ws));
}

}  // namespace

int main(int argc, char** argv) {
  hipStream_t s;
  CK(hipStreamCreate(&s));
  for (const Cfg& c : kCfgs)
    if (argc < 2 || std::strstr(c.name, argv[1])) run(c, s);
  CK(hipStreamDestroy(s));
  return 0;
}
