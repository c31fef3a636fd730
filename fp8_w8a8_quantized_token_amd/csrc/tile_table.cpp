// Per-(kind, N, K) tile-config tables with nearest-M lookup.
//
// The mechanism follows the PR 34331 digest ("Tune FP8 GEMM Triton tiles on
// L40S and enable them by default", sections "Implementation" steps 1, 4, 5
// and "Key source excerpts"): one JSON file per (N, K, device, dtype) whose
// keys are M values; the entry with the key nearest to the requested M wins
// (a tie goes to the smaller key, as a minimum over ascending keys does); a
// null entry, an absent file or an untuned (N, K) keep the default path; the
// file is read once per (N, K); an environment switch turns the tables off.
// Here the device key is the gfx architecture ("gfx950") and the dtype key is
// "fp8_w8a8_channelwise" or "fp8_w8a8_blockwise".
#include "tile_table.h"

#include <dlfcn.h>

#include <algorithm>
#include <cctype>
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

#include "kernels.h"

namespace fp8w8a8 {
namespace {

// ---- a small JSON reader: objects, arrays, strings, numbers, literals ----
struct JVal {
  enum T { Null, Bool, Num, Str, Obj, Arr } t = Null;
  double num = 0;
  bool b = false;
  std::string str;
  std::vector<std::pair<std::string, JVal>> obj;
  std::vector<JVal> arr;
};

struct JParser {
  const char* s;
  const char* e;
  bool ok = true;
  void ws() {
    while (s < e && std::isspace((unsigned char)*s)) ++s;
  }
  bool lit(const char* w) {
    const size_t n = std::strlen(w);
    if ((size_t)(e - s) >= n && std::strncmp(s, w, n) == 0) {
      s += n;
      return true;
    }
    return false;
  }
  std::string str() {
    std::string out;
    if (s >= e || *s != '"') { ok = false; return out; }
    ++s;
    while (s < e && *s != '"') {
      if (*s == '\\' && s + 1 < e) {
        ++s;
        switch (*s) {
          case 'n': out += '\n'; break;
          case 't': out += '\t'; break;
          default: out += *s; break;
        }
        ++s;
      } else {
        out += *s++;
      }
    }
    if (s >= e) { ok = false; return out; }
    ++s;
    return out;
  }
  JVal val() {
    JVal v;
    ws();
    if (s >= e) { ok = false; return v; }
    if (*s == '{') {
      ++s;
      v.t = JVal::Obj;
      ws();
      if (s < e && *s == '}') { ++s; return v; }
      while (ok) {
        ws();
        std::string k = str();
        ws();
        if (s >= e || *s != ':') { ok = false; break; }
        ++s;
        JVal x = val();
        v.obj.emplace_back(std::move(k), std::move(x));
        ws();
        if (s < e && *s == ',') { ++s; continue; }
        if (s < e && *s == '}') { ++s; break; }
        ok = false;
      }
    } else if (*s == '[') {
      ++s;
      v.t = JVal::Arr;
      ws();
      if (s < e && *s == ']') { ++s; return v; }
      while (ok) {
        v.arr.push_back(val());
        ws();
        if (s < e && *s == ',') { ++s; continue; }
        if (s < e && *s == ']') { ++s; break; }
        ok = false;
      }
    } else if (*s == '"') {
      v.t = JVal::Str;
      v.str = str();
    } else if (lit("null")) {
      v.t = JVal::Null;
    } else if (lit("true")) {
      v.t = JVal::Bool; v.b = true;
    } else if (lit("false")) {
      v.t = JVal::Bool; v.b = false;
    } else {
      char* end = nullptr;
      std::string tmp(s, (size_t)std::min<ptrdiff_t>(e - s, 64));
      v.num = std::strtod(tmp.c_str(), &end);
      if (end == tmp.c_str()) { ok = false; return v; }
      v.t = JVal::Num;
      s += (end - tmp.c_str());
    }
    return v;
  }
};

struct Entry {
  int64_t m;
  bool is_null;
  fp8_tile_config cfg;
};

struct Table {
  bool present = false;
  std::vector<Entry> entries;  // ascending m
};

std::mutex g_mu;
std::map<std::tuple<int, int64_t, int64_t>, Table> g_tables;
std::string g_dir_override;
bool g_dir_set = false;

std::string library_dir() {
  Dl_info info;
  if (dladdr(reinterpret_cast<void*>(&library_dir), &info) && info.dli_fname) {
    std::string p(info.dli_fname);
    const size_t slash = p.rfind('/');
    if (slash != std::string::npos) return p.substr(0, slash);
  }
  return ".";
}

std::string config_dir() {
  if (g_dir_set) return g_dir_override;
  const char* env = std::getenv("FP8W8A8_CONFIG_DIR");
  if (env && *env) return env;
  return library_dir() + "/configs";
}

int variant_from_name(const std::string& n) {
  if (n == "skinny") return FP8_VARIANT_SKINNY;
  if (n == "t64x64") return FP8_VARIANT_T64x64;
  if (n == "t128x128") return FP8_VARIANT_T128x128;
  if (n == "t256x128") return FP8_VARIANT_T256x128;
  if (n == "t256x256") return FP8_VARIANT_T256x256;
  if (n == "t256x256w8") return FP8_VARIANT_T256x256W8;
  if (n == "t256x128w8") return FP8_VARIANT_T256x128W8;
  if (n == "t128x128w8") return FP8_VARIANT_T128x128W8;
  if (n == "t128x64k256") return FP8_VARIANT_T128x64K256;
  if (n == "t64x128k256") return FP8_VARIANT_T64x128K256;
  if (n == "t128x128k256") return FP8_VARIANT_T128x128K256;
  if (n == "t256x256dma") return FP8_VARIANT_T256x256DMA;
  if (n == "t256x128dma") return FP8_VARIANT_T256x128DMA;
  if (n == "t128x128dma") return FP8_VARIANT_T128x128DMA;
  if (n == "t256x256panel") return FP8_VARIANT_T256x256PANEL;
  if (n == "t256x128panel") return FP8_VARIANT_T256x128PANEL;
  if (n == "t128x128panel") return FP8_VARIANT_T128x128PANEL;
  if (n == "t128x64panel") return FP8_VARIANT_T128x64PANEL;
  if (n == "t64x64panel") return FP8_VARIANT_T64x64PANEL;
  if (n == "t64x64deep") return FP8_VARIANT_T64x64DEEP;
  if (n == "t128x64deep") return FP8_VARIANT_T128x64DEEP;
  if (n == "t128x128panel8") return FP8_VARIANT_T128x128PANEL8;
  if (n == "t128x64panel8") return FP8_VARIANT_T128x64PANEL8;
  if (n == "t32x32deep") return FP8_VARIANT_T32x32DEEP;
  if (n == "t64x32deep") return FP8_VARIANT_T64x32DEEP;
  if (n == "t256x256bw16") return FP8_VARIANT_T256x256BW16;
  if (n == "decode") return FP8_VARIANT_DECODE;
  return -100;
}

bool parse_table(const std::string& text, Table* t, std::string* err) {
  JParser p{text.data(), text.data() + text.size()};
  JVal root = p.val();
  p.ws();
  if (!p.ok || root.t != JVal::Obj || p.s != p.e) {
    *err = "malformed JSON";
    return false;
  }
  for (auto& kv : root.obj) {
    char* end = nullptr;
    const long long m = std::strtoll(kv.first.c_str(), &end, 10);
    if (end == kv.first.c_str() || *end != '\0' || m < 0) {
      *err = "bad M key '" + kv.first + "'";
      return false;
    }
    Entry en{};
    en.m = m;
    if (kv.second.t == JVal::Null) {
      en.is_null = true;
    } else if (kv.second.t == JVal::Obj) {
      en.is_null = false;
      en.cfg.variant = -100;
      en.cfg.split_k = 1;
      for (auto& f : kv.second.obj) {
        if (f.first == "variant") {
          if (f.second.t == JVal::Str) en.cfg.variant = variant_from_name(f.second.str);
          else if (f.second.t == JVal::Num) en.cfg.variant = (int)f.second.num;
        } else if (f.first == "split_k" && f.second.t == JVal::Num) {
          en.cfg.split_k = (int)f.second.num;
        }
      }
      const VariantInfo vi = variant_info(en.cfg.variant);
      if (!vi.exists || en.cfg.split_k < 1) {
        *err = "bad config at M=" + kv.first;
        return false;
      }
      en.cfg.bm = vi.bm; en.cfg.bn = vi.bn; en.cfg.bk = vi.bk; en.cfg.waves = vi.waves;
    } else {
      *err = "entry for M=" + kv.first + " is neither an object nor null";
      return false;
    }
    t->entries.push_back(en);
  }
  std::sort(t->entries.begin(), t->entries.end(),
            [](const Entry& x, const Entry& y) { return x.m < y.m; });
  t->present = !t->entries.empty();
  return true;
}

const Table& get_table(int kind, int64_t N, int64_t K) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto key = std::make_tuple(kind, N, K);
  auto it = g_tables.find(key);
  if (it != g_tables.end()) return it->second;
  Table t;
  const std::string path = config_dir() + "/N=" + std::to_string(N) + ",K=" + std::to_string(K) +
                           ",device_name=gfx950,dtype=fp8_w8a8_" +
                           (kind == FP8_KIND_BLOCKWISE ? "blockwise" : "channelwise") + ".json";
  std::ifstream f(path);
  if (f) {
    std::stringstream ss;
    ss << f.rdbuf();
    std::string err;
    if (!parse_table(ss.str(), &t, &err)) {
      std::fprintf(stderr, "fp8w8a8: ignoring tile table %s: %s\n", path.c_str(), err.c_str());
      t = Table{};
    } else {
      const char* lg = std::getenv("FP8W8A8_LOG");
      if (lg && *lg && std::strcmp(lg, "0") != 0)
        std::fprintf(stderr, "fp8w8a8: using tile table %s\n", path.c_str());
    }
  }
  return g_tables.emplace(key, std::move(t)).first->second;
}

bool tables_enabled() {
  const char* v = std::getenv("FP8W8A8_TUNED_CONFIGS");
  if (!v) return true;
  std::string s(v);
  for (auto& c : s) c = (char)std::tolower((unsigned char)c);
  return !(s == "0" || s == "false" || s == "off" || s == "no");
}

}  // namespace

int default_config(int kind, int64_t N, int64_t K, int64_t M, fp8_tile_config* out) {
  // Measured on MI355X (o_proj, qkv, down, gate_up and the blockwise shapes,
  // HBM-resident weights): up to 32 rows the decode stream or the
  // register-staged weight stream (below), then,
  // for K % 128 == 0, the panel-ring LDS-DMA tiles: 64x64 up to M = 256 (deep
  // ring for channelwise), 128x64 up to 512 (deep ring for channelwise), the
  // 8-wave 128x128 up to 1024, then 256x128, or 256x256 where it gives at
  // least 192 workgroups (channelwise at M <= 1024 only if it fills all 256
  // compute units; blockwise the 16x16x128-MFMA tile, 8-15% ahead of 256x128
  // at M = 4096-8192). Without that K the register-staged tiles run
  // (channelwise with K % 64 == 0: the 64-byte-stage DMA tiles at large M); a
  // large tile is taken only if it gives at least half the compute units a
  // workgroup, the 64x64 tile being the fallback. Split-K at 32 < M <= 128
  // (64x64 tiles, K % 128 == 0): with at most 128 output tiles and at least 24
  // 128-deep K stages, 2 splits, and 4 with at most 64 tiles and at least 48
  // stages (measured on tabled and untabled shapes, 4096-8192 wide: 10-45%
  // faster there; unsplit stays ahead from ~160 tiles or below ~24 stages).
  const bool cw = kind != FP8_KIND_BLOCKWISE;
  const bool k128 = K % 128 == 0, k64 = cw && K % 64 == 0;
  fp8_tile_config c{};
  c.split_k = 1;
  const int64_t groups = (N + 15) / 16;  // weight-streaming workgroups
  if (M <= 16 && k128 && (groups > 256 ? (M <= 4 || groups < 896) : K >= 6144)) {
    // The LDS-DMA decode stream, measured against the register-staged
    // weight stream and the 32x32 deep-ring tile (HBM-resident weights): with
    // more workgroups than compute units (two share one) ahead everywhere up
    // to ~3.5 rounds (5120^2 9.2-9.5 against 11.5-14.8 us, blockwise 7168^2
    // 13.9-14.7 against 16.6-18.2, qkv 6144x4096 9.1-9.5 against 9.4-11.0)
    // and at M <= 4 beyond (gate_up 24576x4096 22.2 against 25.8); within one
    // round from 6 KB deep rows (down 4096x12288 12.0-13.2 against 13.9-16.6,
    // 4096x7168 8.2-8.7 against 9.2-11.1); on shallower ones (o_proj
    // 4096x4096, 3072x4096) the register-staged stream, 0.3-0.8 us ahead.
    c.variant = FP8_VARIANT_DECODE;
  } else if (M > 16 && M <= 32 && k128 && groups <= 256) {
    // two activation tiles per wave, one round of workgroups: the decode
    // stream again (o_proj 4096x4096 M = 32 7.3 against 8.7 us, down
    // 4096x12288 15.7 against 17.9, blockwise 3072x4096 7.7 against 9.3,
    // 4096x1536 5.6 against 7.9); with more groups its 6 KB slots leave
    // one workgroup per compute unit and it falls behind
    c.variant = FP8_VARIANT_DECODE;
  } else if (M <= 32) {
    c.variant = FP8_VARIANT_SKINNY;
    // From M = 8, on wide weights whose N/16 weight-streaming workgroups run
    // in uneven rounds over the 256 compute units (or N >= 12288), the 32x32
    // deep-ring tile is ahead: 14336x4096 M = 16 15.9 against 19.0 us (decode
    // stream) and 20.4 (register-staged), blockwise 12288x7168 M = 32 20.6
    // against 31.6; 2 splits over 40 or more K stages (blockwise: 24).
    if (M >= 8 && k128 && ((groups > 256 && groups % 256 != 0) || N >= 12288)) {
      c.variant = FP8_VARIANT_T32x32DEEP;
      c.split_k = K / 128 >= (cw ? 40 : 24) ? 2 : 1;
    }
  } else if (k128 && M <= 256) {
    c.variant = cw ? FP8_VARIANT_T64x64DEEP : FP8_VARIANT_T64x64PANEL;
    const int64_t tiles = variant_tiles(c.variant, M, N), stages = K / 128;
    if (M <= 128 && tiles <= 128 && stages >= 24) c.split_k = tiles <= 64 && stages >= 48 ? 4 : 2;
  } else if (k128 && M <= 512) {
    c.variant = cw ? FP8_VARIANT_T128x64DEEP : FP8_VARIANT_T128x64PANEL;
  } else if (k128 && M <= 1024) {
    c.variant = FP8_VARIANT_T128x128PANEL8;
    if (cw && variant_tiles(FP8_VARIANT_T256x256PANEL, M, N) >= 256) c.variant = FP8_VARIANT_T256x256PANEL;
  } else if (k128) {
    c.variant = FP8_VARIANT_T256x128PANEL;
    if (variant_tiles(FP8_VARIANT_T256x256PANEL, M, N) >= 192)
      c.variant = cw ? FP8_VARIANT_T256x256PANEL : FP8_VARIANT_T256x256BW16;
  } else {
    struct Cand {
      int variant;
      int64_t min_tiles;
    };
    Cand order[4];
    int n = 0;
    if (M <= 256) {
      order[n++] = {FP8_VARIANT_T64x64, 128};
    } else if (M <= 512) {
      order[n++] = {FP8_VARIANT_T128x64K256, 128};
    } else if (M <= 1024) {
      order[n++] = {FP8_VARIANT_T128x128K256, 128};
      order[n++] = {FP8_VARIANT_T128x64K256, 128};
    } else {
      if (k64) order[n++] = {FP8_VARIANT_T256x128DMA, 128};
      order[n++] = {FP8_VARIANT_T256x128W8, 128};
      order[n++] = {FP8_VARIANT_T128x128K256, 128};
    }
    c.variant = FP8_VARIANT_T64x64;
    for (int i = 0; i < n; ++i) {
      if (variant_tiles(order[i].variant, M, N) >= order[i].min_tiles) {
        c.variant = order[i].variant;
        break;
      }
    }
  }
  const VariantInfo vi = variant_info(c.variant);
  c.bm = vi.bm; c.bn = vi.bn; c.bk = vi.bk; c.waves = vi.waves;
  *out = c;
  return 0;
}

int lookup_config(int kind, int64_t N, int64_t K, int64_t M, fp8_tile_config* out) {
  if (tables_enabled()) {
    const Table& t = get_table(kind, N, K);
    if (t.present) {
      const Entry* best = &t.entries[0];
      for (const Entry& e : t.entries) {
        const int64_t d = e.m > M ? e.m - M : M - e.m;
        const int64_t db = best->m > M ? best->m - M : M - best->m;
        if (d < db) best = &e;  // strict: ties keep the smaller key
      }
      if (!best->is_null) {
        *out = best->cfg;
        return 1;
      }
    }
  }
  return default_config(kind, N, K, M, out);
}

void set_config_dir(const char* dir) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (dir) {
    g_dir_override = dir;
    g_dir_set = true;
  } else {
    g_dir_override.clear();
    g_dir_set = false;
  }
  g_tables.clear();
}

}  // namespace fp8w8a8
