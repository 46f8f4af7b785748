// Per-shape config table (ai-radar.it, "Helion nel backend vLLM", paragraphs
// 6-7: tuned configs are shipped per shape, with a default config for shapes
// that have none).  Entries are keyed by (arch, abi, fmt, op, weight layout,
// M, N, K), M being the token count T for the MoE ops.  A GEMM or linear
// lookup that misses, or finds only entries written for another arch or ABI
// (kept in the file, never used), falls back to an entry of the same
// floor(log2 M) bucket and then to the cost model's pick (the hard-fallback
// cases of TensorRT-LLM issue 16363, "Suggested direction", that apply to a
// table: cache miss and backend identity mismatch); the MoE ops read exact
// entries only.
#include <cerrno>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>
#include <string>
#include <tuple>
#include <vector>

#include "w8_internal.hpp"

namespace w8 {
namespace {

struct Entry {
  w8_cfg cfg;
  double us;
};

typedef std::tuple<int, int, int, int, int, int> Key;  // fmt, op, layout, M, N, K

const char* layout_name(int layout) {
  switch (layout) {
    case 0: return "row";
    case 1: return "packed";
    case 2: return "seg2";
    case 4: return "seg4";
    case 8: return "seg8";
  }
  return "?";
}
const char* op_name(int op) {
  return op == W8_OP_LINEAR       ? "linear"
         : op == W8_OP_MOE        ? "moe"
         : op == W8_OP_MOE_LINEAR ? "moe_linear"
                                  : "gemm";
}

struct Table {
  std::mutex mu;
  std::map<Key, Entry> native;
  std::vector<std::string> foreign;  // lines for another arch / abi, kept verbatim
  int foreign_count = 0;
  bool env_checked = false;
};

Table& table() {
  static Table t;
  return t;
}

bool parse_int(const std::string& s, int* out) {
  if (s.empty()) return false;
  char* end = nullptr;
  errno = 0;
  long v = std::strtol(s.c_str(), &end, 10);
  if (errno || *end != '\0' || v < -2147483647L || v > 2147483647L) return false;
  *out = (int)v;
  return true;
}

bool parse_double(const std::string& s, double* out) {
  if (s.empty()) return false;
  char* end = nullptr;
  errno = 0;
  double v = std::strtod(s.c_str(), &end);
  if (errno || *end != '\0') return false;
  *out = v;
  return true;
}

// Parses `text`; on success fills native/foreign, else returns the failing
// line number and a reason.
w8_status parse_table(const std::string& text, std::map<Key, Entry>* native,
                      std::vector<std::string>* foreign) {
  std::istringstream in(text);
  std::string line;
  int lineno = 0;
  while (std::getline(in, line)) {
    ++lineno;
    const size_t hash = line.find('#');
    const std::string body = hash == std::string::npos ? line : line.substr(0, hash);
    std::istringstream ls(body);
    std::vector<std::string> tok;
    std::string t;
    while (ls >> t) tok.push_back(t);
    if (tok.empty()) continue;
    const std::string where = "config table line " + std::to_string(lineno) + ": ";
    int abi = 0;
    if (tok.size() < 2 || !parse_int(tok[1], &abi))
      return fail(W8_E_TABLE_FORMAT, where + "expected arch and abi fields");
    // An entry for another arch or ABI (whose fields may differ) is kept verbatim.
    if (tok[0] != kArch || abi != W8_ABI_VERSION) {
      foreign->push_back(line);
      continue;
    }
    if (tok.size() != 18)
      return fail(W8_E_TABLE_FORMAT, where + "expected 18 fields, got " + std::to_string(tok.size()));
    const int fmt = fmt_from_name(tok[2]);
    if (fmt < 0) return fail(W8_E_TABLE_FORMAT, where + "unknown format '" + tok[2] + "'");
    int op = -1;
    if (tok[3] == "gemm") op = W8_OP_GEMM;
    if (tok[3] == "linear") op = W8_OP_LINEAR;
    if (tok[3] == "moe") op = W8_OP_MOE;
    if (tok[3] == "moe_linear") op = W8_OP_MOE_LINEAR;
    if (op < 0)
      return fail(W8_E_TABLE_FORMAT, where + "op must be gemm, linear, moe or moe_linear");
    int packed = -1;  // the weight layout
    for (int l : {0, 1, 2, 4, 8})
      if (tok[4] == layout_name(l)) packed = l;
    if (packed < 0)
      return fail(W8_E_TABLE_FORMAT, where + "layout must be row, packed, seg2, seg4 or seg8");
    int v[12];  // M N K tile_n waves_k waves_n unroll split_k grid swap_ab x_lds quant_launch
    for (int i = 0; i < 12; ++i)
      if (!parse_int(tok[5 + i], &v[i]))
        return fail(W8_E_TABLE_FORMAT, where + "bad integer '" + tok[5 + i] + "'");
    double us = 0;
    if (!parse_double(tok[17], &us)) return fail(W8_E_TABLE_FORMAT, where + "bad time field");
    w8_cfg c;
    std::memset(&c, 0, sizeof c);
    c.abi_version = abi;
    c.tile_n = v[3];
    c.waves_k = v[4];
    c.waves_n = v[5];
    c.unroll = v[6];
    c.split_k = v[7];
    c.grid = v[8];
    c.swap_ab = v[9];
    c.x_lds = v[10];
    c.quant_launch = v[11];
    if (check_gemm_shape(fmt, v[0], v[1], v[2]) != W8_OK ||
        check_cfg(fmt, op, v[0], v[1], v[2], c, packed) != W8_OK)
      return fail(W8_E_TABLE_FORMAT, where + "invalid entry (" + std::string(w8_last_error()) + ")");
    (*native)[Key(fmt, op, packed, v[0], v[1], v[2])] = Entry{c, us};
  }
  return W8_OK;
}

w8_status load_file(const char* path) {
  std::ifstream f(path, std::ios::binary);
  if (!f) return fail(W8_E_IO, std::string("cannot open ") + path);
  std::stringstream ss;
  ss << f.rdbuf();
  if (f.bad()) return fail(W8_E_IO, std::string("cannot read ") + path);
  std::map<Key, Entry> native;
  std::vector<std::string> foreign;
  w8_status st = parse_table(ss.str(), &native, &foreign);
  if (st) return st;
  Table& t = table();
  std::lock_guard<std::mutex> lk(t.mu);
  t.native.swap(native);
  t.foreign.swap(foreign);
  t.foreign_count = (int)t.foreign.size();
  t.env_checked = true;
  return ok();
}

void maybe_load_env(Table& t) {
  // called with t.mu held
  if (t.env_checked) return;
  t.env_checked = true;
  const char* p = std::getenv("W8_CONFIG_TABLE");
  if (!p || !*p) return;
  std::ifstream f(p, std::ios::binary);
  if (!f) return;
  std::stringstream ss;
  ss << f.rdbuf();
  std::map<Key, Entry> native;
  std::vector<std::string> foreign;
  if (parse_table(ss.str(), &native, &foreign) == W8_OK) {
    t.native.swap(native);
    t.foreign.swap(foreign);
    t.foreign_count = (int)t.foreign.size();
  } else if (std::getenv("W8_LOG")) {
    std::fprintf(stderr, "w8gemm: W8_CONFIG_TABLE not loaded: %s\n", w8_last_error());
  }
}

}  // namespace

static int m_bucket(int M) { return 31 - __builtin_clz((unsigned)M); }  // floor(log2 M)

w8_cfg resolve_cfg(int fmt, int op, int M, int N, int K, int layout, int* from_table) {
  Table& t = table();
  {
    std::lock_guard<std::mutex> lk(t.mu);
    maybe_load_env(t);
    const int pk = layout;
    auto it = t.native.find(Key(fmt, op, pk, M, N, K));
    if (it != t.native.end()) {
      if (from_table) *from_table = 1;
      return it->second.cfg;
    }
    // M-bucket fallback (flashinfer-ai/flashinfer pull 3948: the pick is
    // made per floor(log2 M)): the entry of the nearest M in the bucket,
    // the larger on a tie, if its config is valid for this M.
    const int bucket = m_bucket(M);
    const w8_cfg* pick = nullptr;
    int pick_dist = 1 << 30, pick_m = 0;
    for (int m = 1 << bucket; m < (2 << bucket) && m <= W8_MAX_M; ++m) {
      if (m == M) continue;
      auto e = t.native.find(Key(fmt, op, pk, m, N, K));
      if (e == t.native.end()) continue;
      const int d = m > M ? m - M : M - m;
      if (d < pick_dist || (d == pick_dist && m > pick_m)) {
        w8_cfg c = e->second.cfg;
        if (check_cfg(fmt, op, M, N, K, c, layout) != W8_OK) continue;
        pick = &e->second.cfg;
        pick_dist = d;
        pick_m = m;
      }
    }
    if (pick) {
      if (from_table) *from_table = 2;
      return *pick;
    }
  }
  if (from_table) *from_table = 0;
  return model_cfg(fmt, op, M, N, K, layout);
}

}  // namespace w8

using namespace w8;

extern "C" {

w8_status w8_load_config_table(const char* path) {
  if (!path) return fail(W8_E_INVALID, "null path");
  return load_file(path);
}

w8_status w8_save_config_table(const char* path) {
  if (!path) return fail(W8_E_INVALID, "null path");
  std::ostringstream out;
  {
    Table& t = table();
    std::lock_guard<std::mutex> lk(t.mu);
    maybe_load_env(t);
    out << "# w8gemm per-shape config table\n"
        << "# arch abi fmt op layout M N K tile_n waves_k waves_n unroll split_k grid swap_ab "
           "x_lds quant_launch us_per_call\n";
    for (const auto& kv : t.native) {
      const Entry& e = kv.second;
      char buf[256];
      std::snprintf(buf, sizeof buf, "%s %d %s %s %s %d %d %d %d %d %d %d %d %d %d %d %d %.4f\n",
                    kArch, W8_ABI_VERSION, fmt_name(std::get<0>(kv.first)),
                    op_name(std::get<1>(kv.first)), layout_name(std::get<2>(kv.first)),
                    std::get<3>(kv.first), std::get<4>(kv.first), std::get<5>(kv.first),
                    e.cfg.tile_n, e.cfg.waves_k,
                    e.cfg.waves_n, e.cfg.unroll, e.cfg.split_k, e.cfg.grid, e.cfg.swap_ab,
                    e.cfg.x_lds, e.cfg.quant_launch, e.us);
      out << buf;
    }
    for (const auto& l : t.foreign) out << l << "\n";
  }
  // write-then-rename so a crash never leaves a truncated table behind
  const std::string tmp = std::string(path) + ".tmp";
  {
    std::ofstream f(tmp, std::ios::binary | std::ios::trunc);
    if (!f) return fail(W8_E_IO, "cannot write " + tmp);
    f << out.str();
    f.flush();
    if (!f) return fail(W8_E_IO, "write failed: " + tmp);
  }
  if (std::rename(tmp.c_str(), path) != 0) return fail(W8_E_IO, std::string("cannot rename to ") + path);
  return ok();
}

void w8_clear_config_table(void) {
  Table& t = table();
  std::lock_guard<std::mutex> lk(t.mu);
  t.native.clear();
  t.foreign.clear();
  t.foreign_count = 0;
  t.env_checked = true;
}

int w8_config_table_size(void) {
  Table& t = table();
  std::lock_guard<std::mutex> lk(t.mu);
  maybe_load_env(t);
  return (int)t.native.size();
}

int w8_config_table_foreign(void) {
  Table& t = table();
  std::lock_guard<std::mutex> lk(t.mu);
  return t.foreign_count;
}

w8_status w8_set_config(w8_fmt fmt_in, w8_op op_in, int M, int N, int K, int layout,
                        const w8_cfg* cfg, double us_per_call) {
  const int fmt = raw_enum(fmt_in);
  const int op = raw_enum(op_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!cfg) return fail(W8_E_INVALID, "null cfg");
  if (!layout_valid(layout)) return fail(W8_E_INVALID, "weight layout must be 0, 1, 2, 4 or 8");
  st = check_cfg(fmt, op, M, N, K, *cfg, layout);
  if (st) return st;
  Table& t = table();
  std::lock_guard<std::mutex> lk(t.mu);
  maybe_load_env(t);
  t.native[Key(fmt, op, layout, M, N, K)] = Entry{*cfg, us_per_call};
  return ok();
}

w8_status w8_lookup_config(w8_fmt fmt_in, w8_op op_in, int M, int N, int K, int layout, w8_cfg* out,
                           double* us_per_call) {
  const int fmt = raw_enum(fmt_in);
  const int op = raw_enum(op_in);
  w8_status st = check_gemm_shape(fmt, M, N, K);
  if (st) return st;
  if (!out) return fail(W8_E_INVALID, "null output pointer");
  if (op != W8_OP_GEMM && op != W8_OP_LINEAR && op != W8_OP_MOE && op != W8_OP_MOE_LINEAR)
    return fail(W8_E_INVALID, "unknown op");
  Table& t = table();
  std::lock_guard<std::mutex> lk(t.mu);
  maybe_load_env(t);
  auto it = t.native.find(Key(fmt, op, layout, M, N, K));
  if (it == t.native.end()) return fail(W8_E_NOT_FOUND, "no table entry for this shape and layout");
  *out = it->second.cfg;
  if (us_per_call) *us_per_call = it->second.us;
  return ok();
}

}  // extern "C"
