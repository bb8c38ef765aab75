// tern_host.cpp -- host side of the C ABI declared in include/tern.h:
// argument validation, the offline weight relayout (tern_pack / tern_unpack),
// the T-based rung dispatcher with its environment knobs, the rung and kernel
// probes, and the choice of kernel and launch plan per call (the launchers
// live next to their kernels in tern_*.hip, behind tern_internal.h).
//
// Dispatcher: rung map, env-switchable thresholds, one probe per branch and
// env read once per process follow the "NINFER ternary perf-tuning" notes,
// section 2 (rung map and probe), section 5 items 1 and 8 (no silent
// fallback; every scratch counted in the declared workspace) and section 7
// (one launch signature; decode choices frozen per process).
#include <algorithm>
#include <array>
#include <atomic>
#include <cerrno>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <vector>

#include "../../include/tern.h"
#include "tern_internal.h"

namespace {

thread_local std::string g_last_error;

tern_status fail(tern_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tern_status ok() {
  g_last_error.clear();
  return TERN_OK;
}

const char* const kRungNames[TERN_RUNG_COUNT] = {"auto", "gemv", "small_t", "small_t_tiled", "s8"};

const char* const kKernelNames[TERN_KERNEL_COUNT] = {
    "quant_s8",        "quant_s8_row",      "quant_s8_rot",   "gemv_limb",        "gemv_bf16",
    "smallt_resident", "smallt_limb_fused", "smallt_limb_prep", "smallt_limb_tile", "smallt_wave",
    "smallt_tile",     "smallt_tile_reduce", "b16_prefill",   "s8_mma",           "s8_reduce",
    "s8_row",          "s8_acc_export",     "stream_read",    "gemv_t5",          "chain",
    "smallt_narrow"};
static_assert(TERN_KERNEL_COUNT == 21, "one name per kernel id");

// ------------------------------------------------------------ configuration

struct Config {
  bool valid = true;
  std::string error;
  tern_rung forced = TERN_RUNG_AUTO;  // TERN_RUNG
  bool s8_enabled = true;             // TERN_S8
  int s8_min_t = 17;                  // TERN_S8_MIN_T
  int small_t_max = 8;                // TERN_SMALL_T_MAX
  int small_t_tiled_max = 0;          // TERN_SMALL_T_TILED_MAX (0 = unset: s8_min_t - 1)
  bool debug = false;                 // TERN_DEBUG
  int debug_min_t = 1;                // TERN_DEBUG_MIN_T
  long debug_budget = 1000;           // TERN_DEBUG_BUDGET
  int tune_strips = 0;                // TERN_TUNE_STRIPS (0 = heuristic)
  int tune_waves = 0;                 // TERN_TUNE_WAVES (0 = heuristic)
  int tune_s8_bm = 0;                 // TERN_TUNE_S8_BM (0 = heuristic)
  int tune_s8_strips = 0;             // TERN_TUNE_S8_STRIPS (0 = heuristic)
  int tune_s8_raster = 0;             // TERN_TUNE_S8_RASTER: 0 heuristic, 1 plain, 2 xcd
  int tune_kparts = 0;                // TERN_TUNE_KPARTS (0 = heuristic)
  int tune_wn = 0;                    // TERN_TUNE_WN (0 = heuristic)
  int tune_wk = 0;                    // TERN_TUNE_WK (0 = heuristic)
  int tune_depth = 0;                 // TERN_TUNE_DEPTH (0 = heuristic)
  bool gemv_bf16 = false;             // TERN_TUNE_GEMV=bf16: time the bf16-operand gemv kernel (default: limb)
  bool gemv_narrow = false;           // TERN_TUNE_GEMV=narrow: narrow layers at T = 1 on the narrow-layer kernel
  bool t5_lanes = false;              // TERN_TUNE_T5=lanes: resident limbs at T = 5 in two token-lane row blocks
  int smallt_kernel = 0;              // TERN_TUNE_SMALLT: 0 = by shape, 1 = tile, 2 = wave, 3 = limb, 4 = resident, 5 = narrow
  bool limb_unfused = false;          // TERN_TUNE_SMALLT=limb2: limbs by the separate prep kernel
};

bool parse_int(const char* s, long lo, long hi, long* out) {
  if (!s || !*s) return false;
  errno = 0;
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  if (errno || *end != '\0' || v < lo || v > hi) return false;
  *out = v;
  return true;
}

Config read_config() {
  Config c;
  auto bad = [&](const char* name, const char* val) {
    if (c.valid) {
      c.valid = false;
      c.error = std::string("invalid ") + name + "='" + val + "'";
    }
  };
  long v;
  if (const char* s = getenv("TERN_RUNG")) {
    int found = -1;
    for (int i = 0; i < TERN_RUNG_COUNT; ++i)
      if (strcmp(s, kRungNames[i]) == 0) found = i;
    if (found < 0)
      bad("TERN_RUNG", s);
    else
      c.forced = (tern_rung)found;
  }
  if (const char* s = getenv("TERN_S8")) {
    if (parse_int(s, 0, 1, &v))
      c.s8_enabled = v != 0;
    else
      bad("TERN_S8", s);
  }
  if (const char* s = getenv("TERN_S8_MIN_T")) {
    if (parse_int(s, 1, 1L << 30, &v))
      c.s8_min_t = (int)v;
    else
      bad("TERN_S8_MIN_T", s);
  }
  if (const char* s = getenv("TERN_SMALL_T_MAX")) {
    if (parse_int(s, 1, 16, &v))
      c.small_t_max = (int)v;
    else
      bad("TERN_SMALL_T_MAX", s);
  }
  if (const char* s = getenv("TERN_SMALL_T_TILED_MAX")) {
    // the last T before s8: the same threshold as TERN_S8_MIN_T - 1
    if (parse_int(s, 1, (1L << 30) - 1, &v) && v >= c.small_t_max &&
        (!getenv("TERN_S8_MIN_T") || v + 1 == c.s8_min_t)) {
      c.small_t_tiled_max = (int)v;
      c.s8_min_t = (int)v + 1;
    } else {
      bad("TERN_SMALL_T_TILED_MAX", s);
    }
  }
  if (const char* s = getenv("TERN_DEBUG")) {
    if (parse_int(s, 0, 1, &v))
      c.debug = v != 0;
    else
      bad("TERN_DEBUG", s);
  }
  if (const char* s = getenv("TERN_DEBUG_MIN_T")) {
    if (parse_int(s, 1, 1L << 30, &v))
      c.debug_min_t = (int)v;
    else
      bad("TERN_DEBUG_MIN_T", s);
  }
  if (const char* s = getenv("TERN_DEBUG_BUDGET")) {
    if (parse_int(s, 0, 1L << 40, &v))
      c.debug_budget = v;
    else
      bad("TERN_DEBUG_BUDGET", s);
  }
  if (const char* s = getenv("TERN_TUNE_STRIPS")) {
    if (parse_int(s, 0, 4, &v) && v != 3)
      c.tune_strips = (int)v;
    else
      bad("TERN_TUNE_STRIPS", s);
  }
  if (const char* s = getenv("TERN_TUNE_WAVES")) {
    if (parse_int(s, 0, 16, &v))
      c.tune_waves = (int)v;
    else
      bad("TERN_TUNE_WAVES", s);
  }
  if (const char* s = getenv("TERN_TUNE_KPARTS")) {
    if (parse_int(s, 0, 64, &v))
      c.tune_kparts = (int)v;
    else
      bad("TERN_TUNE_KPARTS", s);
  }
  if (const char* s = getenv("TERN_TUNE_WN")) {
    if (parse_int(s, 0, 16, &v))
      c.tune_wn = (int)v;
    else
      bad("TERN_TUNE_WN", s);
  }
  if (const char* s = getenv("TERN_TUNE_WK")) {
    if (parse_int(s, 0, 16, &v))
      c.tune_wk = (int)v;
    else
      bad("TERN_TUNE_WK", s);
  }
  if (const char* s = getenv("TERN_TUNE_DEPTH")) {
    if (parse_int(s, 0, 8, &v) && (v == 0 || v == 2 || v == 4 || v == 8))
      c.tune_depth = (int)v;
    else
      bad("TERN_TUNE_DEPTH", s);
  }
  if (const char* s = getenv("TERN_TUNE_GEMV")) {
    if (strcmp(s, "bf16") == 0)
      c.gemv_bf16 = true;
    else if (strcmp(s, "narrow") == 0)
      c.gemv_narrow = true;
    else if (strcmp(s, "limb") != 0)
      bad("TERN_TUNE_GEMV", s);
  }
  if (const char* s = getenv("TERN_TUNE_T5")) {
    if (strcmp(s, "lanes") == 0)
      c.t5_lanes = true;
    else if (strcmp(s, "rows") != 0)
      bad("TERN_TUNE_T5", s);
  }
  if (const char* s = getenv("TERN_TUNE_SMALLT")) {
    if (strcmp(s, "tile") == 0)
      c.smallt_kernel = 1;
    else if (strcmp(s, "wave") == 0)
      c.smallt_kernel = 2;
    else if (strcmp(s, "limb") == 0)
      c.smallt_kernel = 3;
    else if (strcmp(s, "limb2") == 0) {
      c.smallt_kernel = 3;
      c.limb_unfused = true;
    } else if (strcmp(s, "resident") == 0)
      c.smallt_kernel = 4;
    else if (strcmp(s, "narrow") == 0)
      c.smallt_kernel = 5;
    else
      bad("TERN_TUNE_SMALLT", s);
  }
  if (const char* s = getenv("TERN_TUNE_S8_BM")) {
    if (parse_int(s, 0, 64, &v) && (v == 0 || v == 32 || v == 48 || v == 64))  // tokens per wave tile
      c.tune_s8_bm = (int)v;
    else
      bad("TERN_TUNE_S8_BM", s);
  }
  if (const char* s = getenv("TERN_TUNE_S8_STRIPS")) {
    if (parse_int(s, 0, 4, &v) && (v == 0 || v == 1 || v == 2 || v == 4))
      c.tune_s8_strips = (int)v;
    else
      bad("TERN_TUNE_S8_STRIPS", s);
  }
  if (const char* s = getenv("TERN_TUNE_S8_RASTER")) {
    if (strcmp(s, "plain") == 0)
      c.tune_s8_raster = 1;
    else if (strcmp(s, "xcd") == 0)
      c.tune_s8_raster = 2;
    else
      bad("TERN_TUNE_S8_RASTER", s);
  }
  return c;
}

const Config& config() {
  static std::once_flag once;
  static Config cfg;
  std::call_once(once, [] { cfg = read_config(); });
  return cfg;
}

// ------------------------------------------------------------------- probe

std::atomic<uint64_t> g_probe[TERN_RUNG_COUNT];
std::atomic<uint64_t> g_kprobe[TERN_KERNEL_COUNT];
std::atomic<int> g_last_rung{TERN_RUNG_AUTO};
std::atomic<long> g_debug_lines{0};
thread_local uint64_t t_call_kernels = 0;  // kernels launched by the call in progress
thread_local uint64_t t_last_kernels = 0;  // ... by the last successful call on this thread

// Every entry point that launches opens a call (clears the kernel set) and,
// on success, closes it (publishes the set).
void call_begin() { t_call_kernels = 0; }
tern_status call_ok() {
  t_last_kernels = t_call_kernels;
  g_last_error.clear();
  return TERN_OK;
}

void probe_hit(tern_rung r, int T, int n, int k, int group) {
  g_probe[r].fetch_add(1, std::memory_order_relaxed);
  g_last_rung.store(r, std::memory_order_relaxed);
  const Config& c = config();
  if (c.debug && T >= c.debug_min_t) {
    long i = g_debug_lines.fetch_add(1, std::memory_order_relaxed);
    if (i < c.debug_budget) {
      std::string ks;
      for (int kid = 0; kid < TERN_KERNEL_COUNT; ++kid)
        if (t_call_kernels >> kid & 1) {
          if (!ks.empty()) ks += ',';
          ks += kKernelNames[kid];
        }
      fprintf(stderr, "rung=%s T=%d N=%d K=%d G=%d kernels=%s\n", kRungNames[r], T, n, k, group,
              ks.c_str());
    }
  }
}

// -------------------------------------------------------------- validation

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxK = 1 << 20;
constexpr int kMaxN = 1 << 24;

tern_status check_shape(int n, int k, int group) {
  if (n < 16 || n % 16 != 0)
    return fail(TERN_ERR_SHAPE, "N=%d must be a positive multiple of 16", n);
  if (k < 256 || k % 256 != 0)
    return fail(TERN_ERR_SHAPE, "K=%d must be a positive multiple of 256", k);
  if (group != 64 && group != 128) return fail(TERN_ERR_SHAPE, "G=%d must be 64 or 128", group);
  // The kernels form activation offsets inside a tile of up to 128 rows and
  // the bytes of up to 16 strips of codes in 32 bits, and s8 grids of
  // N/256 x T/32 workgroups: K <= 2^20 and N <= 2^24 keep all of them in range.
  if (k > kMaxK) return fail(TERN_ERR_SHAPE, "K=%d above the supported %d", k, kMaxK);
  if (n > kMaxN) return fail(TERN_ERR_SHAPE, "N=%d above the supported %d", n, kMaxN);
  return TERN_OK;
}

constexpr int kMaxTokens = 1 << 19;  // keeps every grid y dimension below 65536

// Resolve the rung for a call. Returns TERN_OK and sets *out, or an error.
tern_status resolve(int T, tern_rung req, tern_rung* out) {
  const Config& c = config();
  if (!c.valid) return fail(TERN_ERR_CONFIG, "%s", c.error.c_str());
  if ((int)req < 0 || (int)req >= TERN_RUNG_COUNT)
    return fail(TERN_ERR_RUNG, "unknown rung %d", (int)req);
  if (T < 1 || T > kMaxTokens) return fail(TERN_ERR_SHAPE, "T=%d out of range [1, %d]", T, kMaxTokens);
  tern_rung r = req;
  if (r == TERN_RUNG_AUTO) r = c.forced;
  if (r == TERN_RUNG_AUTO) {
    if (c.s8_enabled && T >= c.s8_min_t)
      r = TERN_RUNG_S8;
    else if (T == 1)
      r = TERN_RUNG_GEMV;
    else if (T <= c.small_t_max)
      r = TERN_RUNG_SMALL_T;
    else
      r = TERN_RUNG_SMALL_T_TILED;
  }
  if (r == TERN_RUNG_GEMV && T > 65535)
    return fail(TERN_ERR_RUNG, "rung gemv runs one token per grid row: T=%d > 65535", T);
  if (r == TERN_RUNG_SMALL_T && T > 16)
    return fail(TERN_ERR_RUNG, "rung small_t takes one 16-token tile: T=%d > 16", T);
  *out = r;
  return TERN_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Launch shape of the activation-tiled kernel (small_t, small_t_tiled), from
// sweeps on MI355X over (S, Ws, Pk, D) at T = 4..16: one strip per wave;
// wide layers (N >= 16k) take 4 compute waves per workgroup, no K split and
// 2 k-tiles in flight (67 VGPRs, 7 waves per SIMD), narrower ones 8 waves, K
// split 4 ways (partials through the workspace) and 4 k-tiles in flight.
// Deeper rings cost occupancy and were slower on both.
tern::TilePlan plan_tile(int T, int n, int k) {
  const Config& c = config();
  tern::TilePlan p;
  const int NS = n / 16, KT = k / 256;
  const bool wide = NS >= 1024;
  p.rows = T <= 8 ? 8 : 16;
  p.strips_per_wave = c.tune_strips ? c.tune_strips : 1;
  int Ws = c.tune_waves ? c.tune_waves : (wide ? 4 : 8);
  Ws = std::min(Ws, 8);  // launch bounds
  p.waves = Ws;
  int D = c.tune_depth ? c.tune_depth : (wide ? 2 : 4);
  while (D > 2 && p.strips_per_wave * D > 8) D /= 2;  // code registers: S * D <= 8
  p.depth = D;
  p.token_tiles = (T + 15) / 16;
  p.strip_blocks = (NS + Ws * p.strips_per_wave - 1) / (Ws * p.strips_per_wave);
  int Pk = c.tune_kparts ? c.tune_kparts : (wide ? 1 : 4);
  p.k_parts = std::max(1, std::min(Pk, KT));
  return p;
}

// Kernel of the small_t / small_t_tiled rungs, from A/B runs on MI355X over
// T = 2..16: wide layers (>= 1024 strips) run the activation-tiled kernel;
// narrow ones give it too few workgroups and run the narrow-layer kernel
// (small_t_narrow) or, where that loses, the per-wave kernel (each wave loads
// its own activation fragments, no barriers).
// The small_t limb path (tern_limbtile.hip) takes T <= 8; by default it runs
// wide layers (>= 1024 strips) at T <= 4, one row block, where the resident
// limb kernel (checked first) does not fit its LDS (long K): there it beat
// the bf16 activation-tiled kernel in A/B runs on MI355X (gate_up: 14.0-15.3
// against 15.9-16.6 us); at T = 5..8 (two row blocks) and on narrow layers it
// lost.
bool small_t_limb(int T, int n, int k) {
  (void)k;
  const Config& c = config();
  if (c.smallt_kernel) return c.smallt_kernel == 3 && T <= 8;
  return T <= 4 && n / 16 >= 1024;
}

tern::LimbTilePlan plan_limbtile(int T, int n, int k) {
  (void)k;
  const Config& c = config();
  tern::LimbTilePlan p;
  const int NS = n / 16;
  p.strips_per_wave = c.tune_strips == 2 ? 2 : 1;
  p.waves = c.tune_waves ? std::min(c.tune_waves, 8) : 4;
  // two strips per wave keep 2 k-tiles in flight (4 would spill registers)
  p.depth = c.tune_depth == 4 && p.strips_per_wave == 1 ? 4 : 2;
  p.strip_blocks = (NS + p.waves * p.strips_per_wave - 1) / (p.waves * p.strips_per_wave);
  // Up to 4 tokens the loader wave makes the limbs (one launch, no workspace).
  p.fused = T <= 4 && !c.limb_unfused;
  return p;
}

tern::LimbPlan plan_limb(int T, int n, int k);
int wide_waves(int NS);

// small_t on T <= 8 tokens through the gemv kernel's layout (the limbs of
// the whole K made once per workgroup and kept in LDS, lane group u = tokens
// u and 4 + u, the gemv's work split). By default at T <= 3 where the limbs
// take at most 112 KiB of LDS: there making them up front beats both the
// loader-wave pipeline (wide layers) and the per-wave bf16 kernel (narrow
// ones); at T = 4, or with down's 157 KB at T = 3, the up-front work and the
// LDS lose (A/B on the part). Needs no workspace. The LDS holds the limbs and
// the workgroup's scales, which take twice the bytes at G = 64, so every LDS
// check takes the call's group size.
tern::LimbPlan plan_resident(int T, int n, int k, int G) {
  tern::LimbPlan p = plan_limb(T, n, k);
  p.resident = true;
  // Five tokens fill one 16-row operand as rows 3t + L with per-row totals
  // (the kernel's TT = 5 mode); more need the token-lane mode's second
  // operand. TERN_TUNE_T5=lanes keeps T = 5 on the token lanes.
  p.token_lanes = !(T == 5 && !config().t5_lanes);
  const int NS = n / 16;
  // narrow layers with a long K keep 8 K shares here (the gemv's 6 measured
  // 1 % slower at T = 2 on down)
  if (NS < 1024 && !config().tune_wk && k / 256 >= 48) {
    p.wk = 8;
    while (p.wn * p.wk > 16) --p.wn;
  }
  // Wide layers: the gemv's wide workgroups (one round, one per CU: at
  // T = 2..4 on gate_up, twelve waves, 10.5-10.8 us against 12.0-17.9 with
  // four waves, whose 544 workgroups of 36-78 KB of LDS need up to three
  // rounds), fewer waves where the LDS would not hold them, but never fewer
  // than one round of one workgroup per CU needs.
  if (p.wk == 1 && NS >= 1024 && !config().tune_wn) {
    p.wn = wide_waves(NS);
    const int floor_wn = (NS + 255) / 256;
    while (p.wn > floor_wn && tern::limb_lds_bytes(T, k, G, p) > tern::kLimbMaxLdsResident) --p.wn;
  } else if (p.wk == 1 && tern::limb_lds_bytes(T, k, G, p) > 80 * 1024) {
    // Limbs of more than 80 KiB leave room for one workgroup per CU: make it
    // wide enough that one round of workgroups covers the strips.
    p.wn = std::min(16, std::max(p.wn, (NS + 255) / 256));
  }
  return p;
}

bool small_t_resident(int T, int n, int k, int G) {
  const Config& c = config();
  const int lds = tern::limb_lds_bytes(T, k, G, plan_resident(T, n, k, G));
  if (c.smallt_kernel) return c.smallt_kernel == 4 && T <= 8 && lds <= tern::kLimbMaxLdsResident;
  if (T <= 3) return lds <= 112 * 1024;
  // Wide layers in one round of twelve-wave workgroups: ahead of the fused
  // limb kernel at T = 4 (10.8 against 14.2 us on gate_up) and, with two row
  // blocks of tokens, of the bf16 tile kernel at T = 5..8 (gate_up at T = 7:
  // 16.4-16.5 against 17.2-17.4 us, T = 8: 16.9-17.1 against 17.2-17.4, A/B
  // in one run on MI355X).
  return T <= 8 && n / 16 >= 1024 && lds <= tern::kLimbMaxLdsResident;
}

bool small_t_per_wave(int T, int n, int k) {
  const Config& c = config();
  if (c.smallt_kernel) return c.smallt_kernel == 2;
  return n / 16 < 1024 && (T <= 8 || k <= 8192);
}

tern::S8Plan plan_s8(int T, int n, int k, bool allow_split);

// The narrow-layer kernel (tern_narrow.hip): layers of fewer than 1024
// strips at T <= 16, each workgroup one block of W strips over one of Pk K
// parts, the parts added in the same launch. Pk makes about one workgroup
// per CU (256); every part's k-tiles must fit the wave's register ring. A/B
// on MI355X (graphs of 100 calls, weights rotated past the Infinity Cache):
// on down (68 k-tiles) 10.2-11.1 us over T = 3..16 against 11.8-13.8 for the
// per-wave kernel (T <= 8) and the K-split tile kernel with its reduce launch
// (T > 8); down at T = 2 keeps the resident limbs (9.4 against 10.1). On
// o_proj (20 k-tiles) the arrival protocol (about 1.7 us: the partials'
// stores, the count, the last part's loads) outweighs the gain up to
// T = 12 (per-wave kernel 5.9-7.2 us against 6.7-7.2), and wins above
// (7.4 against 8.0 at T = 16).
bool small_t_narrow(int T, int n, int k) {
  const Config& c = config();
  if (c.smallt_kernel) return c.smallt_kernel == 5 && T <= 16;
  if (n / 16 >= 1024 || T > 16) return false;
  return (k / 256 >= 48 && T >= 3) || T >= 13;
}

tern::NarrowPlan plan_narrow(int T, int n, int k) {
  const Config& c = config();
  tern::NarrowPlan p;
  const int NS = n / 16, KT = k / 256;
  p.rows = T <= 4 ? 4 : T <= 8 ? 8 : 16;
  p.waves = c.tune_waves == 16 ? 16 : 8;
  p.strip_blocks = (NS + p.waves - 1) / p.waves;
  int Pk = c.tune_kparts ? c.tune_kparts : (int)std::lround(256.0 / p.strip_blocks);
  Pk = std::max(1, std::min(Pk, KT));
  const int kcap = p.waves == 16 ? 12 : 16;  // registers: 16 waves leave each 128 VGPRs
  while ((KT + Pk - 1) / Pk > kcap) ++Pk;
  if (p.strip_blocks > 1024) Pk = 1;  // one counter per strip block in the workspace header
  const int per = (KT + Pk - 1) / Pk;
  p.kmax = per <= 4 ? 4 : per <= 8 ? 8 : per <= 12 ? 12 : 16;
  p.k_parts = Pk;
  // 4 k-tiles in flight per wave, against all of them requested up front:
  // down 10.1-11.1 against 11.5-12.6 us (a wave's k-tiles then arrive
  // spread out, so its arithmetic overlaps the stream); the same where a
  // part has at most 4 k-tiles (o_proj). TERN_TUNE_DEPTH=2/8 asks for all up front.
  p.depth = c.tune_depth && c.tune_depth != 4 ? 0 : 4;
  return p;
}

// small_t_tiled above one 16-token tile runs the bf16 prefill contraction
// (tern_b16mma.hip), which needs no workspace.
bool b16_prefill(int T, tern_rung r) { return r == TERN_RUNG_SMALL_T_TILED && T > 16; }

tern::SmallTPlan plan_small_t(int T, int n, int k, int group, tern_rung r) {
  (void)group;
  const Config& c = config();
  tern::SmallTPlan p;
  const int NS = n / 16, KT = k / 256;
  int S = 2;
  if (T > 1 && r != TERN_RUNG_GEMV && NS >= 1024) S = 4;
  if (c.tune_strips) S = c.tune_strips;
  // gemv stages the token row in LDS; rows too long for that take the
  // 16-token kernel (its absent rows read as zeros).
  const bool row_in_lds = r == TERN_RUNG_GEMV && tern::small_t_max_waves(1, S, k) >= 1;
  p.tokens_per_tile = row_in_lds ? 1 : 16;
  p.token_tiles = row_in_lds ? T : (T + 15) / 16;
  const int nsb = (NS + S - 1) / S;
  // About 4.3k waves in flight (4 per SIMD) fill the chip in one round for
  // every layer shape measured; the sweep over (S, W) on MI355X picked S = 2
  // everywhere except wide 16-token tiles (S = 4, which share the activation
  // fragments across more strips).
  int W = (int)(4352.0 / (double)(nsb * (long)std::max(1, p.token_tiles)) + 0.5);
  if (p.tokens_per_tile == 16 && !c.tune_strips) W = 4;
  const int wmax = std::max(1, tern::small_t_max_waves(p.tokens_per_tile, S, k));
  W = std::max(1, std::min(W, std::min(wmax, KT)));
  if (c.tune_waves) W = std::max(1, std::min(std::min(c.tune_waves, wmax), KT));
  p.strips_per_wave = S;
  p.waves = W;
  return p;
}

// Launch shape of the integer-limb decode kernel, from sweeps on MI355X at
// T = 1 over (waves per strip group, K shares, ring depth): wide layers (>= 1024
// strips) take one strip per wave over the whole K and NS / 136 waves per
// workgroup, 4 to 12, so that the workgroups make one round of one per CU:
// 2176 strips take 12 waves and 182 workgroups (10.2 us against 11.0 with four
// waves and 544 workgroups, up to three per CU; 8 waves give 272 workgroups
// and a second round, 16 waves too few CUs), 1088 strips 8 waves and 136
// workgroups (7.6 us; 8.4 with four waves, 9.3 with twelve);
// narrow layers two strips per workgroup with K split 6 ways (K >= 12288;
// 12 waves, down 8.4 us against 8.7 with 8 ways) or 4 ways, so that the few strips still give every SIMD several waves. Every
// wave keeps 4 k-tiles of codes in flight. Wide layers whose limbs and
// scales would not fit the kernel's LDS take fewer waves.
int wide_waves(int NS) { return std::min(12, std::max(4, NS / 136)); }

tern::LimbPlan plan_limb(int T, int n, int k) {
  const Config& c = config();
  tern::LimbPlan p;
  const int NS = n / 16, KT = k / 256;
  const bool wide = NS >= 1024;
  p.strips_per_wave = 1;  // the limb kernel is built for one strip per wave only
  p.wn = c.tune_wn ? c.tune_wn : (wide ? wide_waves(NS) : 2);
  p.wk = c.tune_wk ? c.tune_wk : (wide ? 1 : (KT >= 48 ? 6 : 4));
  p.wk = std::min(p.wk, KT);
  while (p.wn * p.wk > 16) --p.wn;
  p.depth = c.tune_depth ? c.tune_depth : (p.strips_per_wave == 1 ? 4 : 2);
  // (the scales of the workgroup's strips share the LDS with the limbs;
  // G = 64 is the larger of the two)
  if (wide && !c.tune_wn)
    while (p.wn > 4 && tern::limb_lds_bytes(T, k, 64, p) > tern::kLimbMaxLds) --p.wn;
  return p;
}

// The integer-limb kernel takes T <= 5 with its activation limbs in LDS.
bool limb_fits(int T, int k, int group, const tern::LimbPlan& p) {
  return T <= 5 && tern::limb_lds_bytes(T, k, group, p) <= tern::kLimbMaxLds;
}

tern::S8Plan plan_s8(int T, int n, int k, bool allow_split) {
  const Config& c = config();
  tern::S8Plan p;
  // Wave tile 64 tokens x 64 outputs (4 token blocks x 4 strips) where that
  // still gives at least 4 workgroups per CU; 64 x 32 otherwise (narrow
  // layers); 32- and 48-token tiles for T <= 32 and T <= 48 so padded tokens
  // do not waste the matrix cores, and one strip per wave up to T = 64, where the kernel is
  // bound by load latency and wants as many waves streaming as it can get.
  // (128-token tiles cost registers, and occupancy, without paying back on
  // either 27B-class shape; they spilled and are not built.)
  const int tb = c.tune_s8_bm ? c.tune_s8_bm / 16 : (T > 48 ? 4 : T > 32 ? 3 : 2);
  const long tiles4 = (long)((n / 16 + 15) / 16) * ((T + 16 * tb - 1) / (16 * tb));
  int strips = T <= 64 ? 1 : (tiles4 >= 1024 ? 4 : 2);
  if (c.tune_s8_strips) strips = c.tune_s8_strips;
  p.token_blocks = tb;
  p.strips = strips;
  p.xcd_order = c.tune_s8_raster != 1;
  // Short prefills on narrow layers give too few tiles to keep HBM busy:
  // split K over workgroups (each part at least 6 k-tiles). With fewer tiles
  // than CUs, into as many parts as keep the grid within 512 workgroups (two
  // per CU, one round: a 513th would start a second round); with fewer than
  // 512 tiles and a long K, into enough parts for about 512. The parts cost a
  // second kernel, which only pays there (A/B runs on MI355X at T =
  // 17..508). Short prefills also keep 3 k-tiles in flight instead of 1.
  const int KT = k / 256;
  auto tiles_for = [&](int st) {
    return (long)((n / 16 + 4 * st - 1) / (4 * st)) * ((T + 16 * tb - 1) / (16 * tb));
  };
  auto parts_for = [&](long tiles) {
    int pk = 1;
    if (allow_split && tiles < 256)
      pk = (int)std::min<long>(512 / tiles, 16);
    else if (allow_split && tiles < 512 && KT >= 32)
      pk = (int)std::min<long>((512 + tiles - 1) / tiles, 16);
    return std::max(1, std::min(pk, KT / 6));  // parts of at least 6 k-tiles (o_proj: 3 parts beat 5 by 6-17 %)
  };
  // Share of the workgroup slots (512 per round) a grid of w workgroups fills.
  auto fill = [](long w) { return (double)w / (512.0 * (double)((w + 511) / 512)); };
  int pk = parts_for(tiles_for(strips));
  // A split that fills its last round poorly: 4 strips per wave, with its own
  // split, when that fills the rounds better (down at T = 508: 640
  // workgroups in 2 parts against 480 in 3, 87 -> 79 us).
  if (!c.tune_s8_strips && strips == 2 && pk > 1) {
    const int pk4 = parts_for(tiles_for(4));
    if (fill(tiles_for(4) * pk4) > fill(tiles_for(2) * pk)) {
      strips = 4;
      pk = pk4;
      p.strips = strips;
    }
  }
  if (c.tune_kparts && allow_split) pk = std::max(1, std::min(c.tune_kparts, KT));
  p.k_parts = pk;
  p.depth = (T <= 64 || pk > 1) ? 4 : 2;
  if (c.tune_depth == 2 || c.tune_depth == 4) p.depth = c.tune_depth;
  // the 64 x 64 and 32 x 64 wave tiles run double-buffered only (registers)
  if (tb * strips >= 16 || (tb == 2 && strips == 4)) p.depth = 2;
  return p;
}

// ------------------------------------------------------- kernel choice

// What one tern_linear call runs, from its resolved rung and the layer shape:
// the path (one kernel, or a pair with its reduction or preparation), the
// launch plan, the workspace it needs and the ids of the kernels it launches.
// tern_linear, tern_workspace_bytes and tern_plan_kernels all take it from
// here, so the declared workspace and the kernel probe's expectations are the
// launch's own.
enum class Path { S8, GEMV_LIMB, PER_WAVE, RESIDENT, LIMBTILE, B16_PREFILL, TILE, NARROW };

struct Choice {
  Path path = Path::S8;
  tern::LimbPlan limb{};          // GEMV_LIMB, RESIDENT
  tern::SmallTPlan wave{};        // PER_WAVE (also the gemv's bf16 kernel)
  tern::LimbTilePlan limbtile{};  // LIMBTILE
  tern::TilePlan tile{};          // TILE
  tern::NarrowPlan narrow{};      // NARROW
  tern::S8Plan s8{};              // S8, B16_PREFILL
  size_t workspace = 0;
  uint64_t kernels = 0;
};

constexpr uint64_t kbit(tern_kernel id) { return uint64_t{1} << id; }

Choice choose_path(int T, int n, int k, int G, tern_rung r) {
  Choice c;
  if (r == TERN_RUNG_S8) {
    c.path = Path::S8;
    c.s8 = plan_s8(T, n, k, true);
    c.workspace = align256((size_t)T * k) + align256((size_t)T * sizeof(float)) +
                  tern::s8_partial_bytes(c.s8, T, n);
    c.kernels = kbit(TERN_KERNEL_QUANT_S8) | kbit(TERN_KERNEL_S8_MMA) |
                (c.s8.k_parts > 1 ? kbit(TERN_KERNEL_S8_REDUCE) : 0);
    return c;
  }
  auto per_wave = [&] {
    c.path = Path::PER_WAVE;
    c.wave = plan_small_t(T, n, k, G, r);
    c.kernels = kbit(c.wave.tokens_per_tile == 1 ? TERN_KERNEL_GEMV_BF16 : TERN_KERNEL_SMALLT_WAVE);
  };
  auto narrow = [&] {
    c.path = Path::NARROW;
    c.narrow = plan_narrow(T, n, k);
    c.workspace = tern::narrow_partial_bytes(c.narrow, T, n);
    c.kernels = kbit(TERN_KERNEL_SMALLT_NARROW);
  };
  if (r == TERN_RUNG_GEMV) {
    if (config().gemv_narrow && n / 16 < 1024) {
      narrow();
      return c;
    }
    c.limb = plan_limb(T, n, k);
    if (!config().gemv_bf16 && limb_fits(T, k, G, c.limb)) {
      c.path = Path::GEMV_LIMB;
      c.kernels = kbit(TERN_KERNEL_GEMV_LIMB);
    } else {
      per_wave();  // limbs and scales beyond the kernel's LDS (or TERN_TUNE_GEMV=bf16)
    }
    return c;
  }
  // small_t and small_t_tiled
  if (small_t_narrow(T, n, k)) {
    narrow();
  } else if (small_t_resident(T, n, k, G)) {
    c.path = Path::RESIDENT;
    c.limb = plan_resident(T, n, k, G);
    c.kernels = kbit(TERN_KERNEL_SMALLT_RESIDENT);
  } else if (small_t_limb(T, n, k)) {
    c.path = Path::LIMBTILE;
    c.limbtile = plan_limbtile(T, n, k);
    if (c.limbtile.fused) {
      c.kernels = kbit(TERN_KERNEL_SMALLT_LIMB_FUSED);
    } else {
      c.workspace = tern::limbtile_workspace_bytes(T, k);
      c.kernels = kbit(TERN_KERNEL_SMALLT_LIMB_PREP) | kbit(TERN_KERNEL_SMALLT_LIMB_TILE);
    }
  } else if (b16_prefill(T, r)) {
    c.path = Path::B16_PREFILL;
    c.s8 = plan_s8(T, n, k, false);
    c.kernels = kbit(TERN_KERNEL_B16_PREFILL);
  } else if (small_t_per_wave(T, n, k)) {
    per_wave();
  } else {
    c.path = Path::TILE;
    c.tile = plan_tile(T, n, k);
    c.workspace = tern::tile_workspace_bytes(c.tile, n);
    c.kernels = kbit(TERN_KERNEL_SMALLT_TILE) |
                (c.tile.k_parts > 1 ? kbit(TERN_KERNEL_SMALLT_TILE_REDUCE) : 0);
  }
  return c;
}

// Every workspace starts with a header of kWsHeader bytes that only the
// narrow-layer kernel uses (its arrival counters, zero on entry and on exit);
// the other paths' scratch follows it, so a workspace shared by calls of
// different paths keeps the counters intact.
constexpr size_t kWsHeader = 4096;
static_assert(kWsHeader >= 1024 * sizeof(int), "a counter per strip block of a narrow layer (< 1024 strips)");

Choice choose(int T, int n, int k, int G, tern_rung r) {
  Choice c = choose_path(T, n, k, G, r);
  if (c.workspace) c.workspace += kWsHeader;
  return c;
}

// The same for base-3 (t5) weights: the gemv rung only, on the limb kernel,
// with the plan of the 2-bit layout; an error for any other rung (a forced
// rung never falls back) or a K whose limbs do not fit the kernel's LDS.
tern_status choose_t5(int T, int n, int k, int G, tern_rung r, Choice* out) {
  if (r != TERN_RUNG_GEMV)
    return fail(TERN_ERR_LAYOUT, "layout t5 runs on the gemv rung only (T = %d resolves to %s)", T,
                kRungNames[r]);
  if (T != 1) return fail(TERN_ERR_LAYOUT, "layout t5 takes one token, T = %d", T);
  Choice c;
  c.path = Path::GEMV_LIMB;
  c.limb = plan_limb(T, n, k);
  c.limb.t5 = true;
  if (tern::limb_lds_bytes(T, k, G, c.limb) > tern::kLimbMaxLds)
    return fail(TERN_ERR_SHAPE, "layout t5: K=%d needs more LDS than the gemv kernel has", k);
  c.kernels = kbit(TERN_KERNEL_GEMV_T5);
  *out = c;
  return TERN_OK;
}

tern_status hip_fail(int err, const char* what) {
  return fail(TERN_ERR_HIP, "%s: %s", what, tern::hip_error_string(err));
}

tern_status check_weights(const tern_weights* W) {
  if (!W) return fail(TERN_ERR_NULL, "W is NULL");
  if (!W->codes || !W->scales) return fail(TERN_ERR_NULL, "W->codes or W->scales is NULL");
  if (W->layout != TERN_LAYOUT_V1 && W->layout != TERN_LAYOUT_T5)
    return fail(TERN_ERR_LAYOUT, "W->layout=0x%08x is neither TERN_LAYOUT_V1 nor TERN_LAYOUT_T5", W->layout);
  tern_status st = check_shape(W->n, W->k, W->group);
  if (st != TERN_OK) return st;
  if (W->layout == TERN_LAYOUT_T5 && W->k % 1024 != 0)
    return fail(TERN_ERR_SHAPE, "layout t5: K=%d must be a multiple of 1024", W->k);
  if (!aligned16(W->codes) || !aligned16(W->scales))
    return fail(TERN_ERR_ALIGN, "W->codes / W->scales must be 16-byte aligned");
  return TERN_OK;
}

inline uint32_t encode(int8_t v) { return v == 0 ? 0u : (v == 1 ? 1u : 3u); }

// tern_linear and tern_linear_noalloc: validate everything on the host, then
// (noalloc: with the device's static scratch as the workspace) launch.
tern_status linear_call(const void* x_bf16, int T, const tern_weights* W, float* y, tern_rung rung,
                        void* ws, size_t ws_bytes, void* stream, bool noalloc) {
  if (!x_bf16 || !y) return fail(TERN_ERR_NULL, "tern_linear: x or y is NULL");
  tern_status st = check_weights(W);
  if (st != TERN_OK) return st;
  if (!aligned16(x_bf16) || !aligned16(y))
    return fail(TERN_ERR_ALIGN, "x and y must be 16-byte aligned");
  tern_rung r;
  st = resolve(T, rung, &r);
  if (st != TERN_OK) return st;
  const int n = W->n, k = W->k, G = W->group;
  Choice c;
  if (W->layout == TERN_LAYOUT_T5) {
    st = choose_t5(T, n, k, G, r, &c);
    if (st != TERN_OK) return st;
  } else {
    c = choose(T, n, k, G, r);
  }
  if (noalloc && c.workspace > ws_bytes)
    return fail(TERN_ERR_WORKSPACE,
                "rung %s needs %zu bytes of workspace, more than the %zu of the static scratch",
                kRungNames[r], c.workspace, ws_bytes);
  if (noalloc && c.workspace) {
    const int err = tern::noalloc_scratch(&ws);  // the device address of this GPU's copy
    if (err) return hip_fail(err, "static scratch lookup");
  }
  if (c.workspace) {
    if (!ws || ws_bytes < c.workspace)
      return fail(TERN_ERR_WORKSPACE, "rung %s needs %zu bytes of workspace, got %zu%s",
                  kRungNames[r], c.workspace, ws ? ws_bytes : (size_t)0, ws ? "" : " (NULL)");
    if (!aligned16(ws)) return fail(TERN_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  const tern::SmallTArgs a{(const uint16_t*)x_bf16, T, k, n, G, W->codes, W->scales, y};
  // the paths' scratch follows the counter header
  char* const wsb = c.workspace ? (char*)ws + kWsHeader : nullptr;
  int err = 0;
  switch (c.path) {
    case Path::S8: {
      int8_t* q = (int8_t*)wsb;
      float* sc = (float*)(wsb + align256((size_t)T * k));
      err = tern::launch_quant_s8((const uint16_t*)x_bf16, T, k, q, sc, true, stream);
      if (err) return hip_fail(err, "quant_s8 launch");
      float* part = (float*)(wsb + align256((size_t)T * k) + align256((size_t)T * sizeof(float)));
      const tern::S8Args sa{q, sc, T, k, n, G, W->codes, W->scales, y, nullptr, true};
      err = tern::launch_s8(sa, c.s8, part, stream);
      if (err) return hip_fail(err, "s8 launch");
      break;
    }
    case Path::GEMV_LIMB:
    case Path::RESIDENT:
      err = tern::launch_limb(a, c.limb, stream);
      if (err) return hip_fail(err, c.path == Path::RESIDENT ? "small_t resident launch" : "gemv launch");
      break;
    case Path::PER_WAVE:
      err = tern::launch_small_t(a, c.wave, stream);
      if (err) return hip_fail(err, r == TERN_RUNG_GEMV ? "gemv launch" : "small_t launch");
      break;
    case Path::LIMBTILE:
      err = tern::launch_limbtile(a, c.limbtile, wsb, stream);
      if (err) return hip_fail(err, "small_t limb launch");
      break;
    case Path::B16_PREFILL:
      err = tern::launch_b16_prefill(a, c.s8, stream);
      if (err) return hip_fail(err, "bf16 prefill launch");
      break;
    case Path::TILE:
      err = tern::launch_tile(a, c.tile, wsb, stream);
      if (err) return hip_fail(err, "small_t launch");
      break;
    case Path::NARROW:
      err = tern::launch_narrow(a, c.narrow, wsb, c.workspace ? (int*)ws : nullptr, stream);
      if (err) return hip_fail(err, r == TERN_RUNG_GEMV ? "gemv launch" : "small_t launch");
      break;
  }
  probe_hit(r, T, n, k, G);
  return call_ok();
}


}  // namespace

int tern::kernel_launched(int err, tern_kernel k) {
  if (err == 0 && (int)k >= 0 && (int)k < TERN_KERNEL_COUNT) {
    g_kprobe[k].fetch_add(1, std::memory_order_relaxed);
    t_call_kernels |= uint64_t{1} << k;
  }
  return err;
}

extern "C" {

int tern_abi_version(void) { return 1; }

const char* tern_last_error(void) { return g_last_error.c_str(); }

const char* tern_rung_name(tern_rung rung) {
  if ((int)rung < 0 || (int)rung >= TERN_RUNG_COUNT) return "invalid";
  return kRungNames[rung];
}

size_t tern_packed_code_bytes(int n, int k) {
  if (n < 16 || n % 16 || k < 256 || k % 256) return 0;
  return (size_t)n * (size_t)k / 4;
}

size_t tern_scale_count(int n, int k, int group) {
  if (check_shape(n, k, group) != TERN_OK) return 0;
  return (size_t)n * (size_t)(k / group);
}

tern_status tern_pack(const int8_t* w, const uint16_t* scales_f16, int n, int k, int group,
                      void* codes_out, uint16_t* scales_out) {
  if (!w || !scales_f16 || !codes_out || !scales_out)
    return fail(TERN_ERR_NULL, "tern_pack: NULL pointer");
  tern_status st = check_shape(n, k, group);
  if (st != TERN_OK) return st;
  const size_t NS = (size_t)n / 16, KT = (size_t)k / 256, GPT = 256 / (size_t)group;
  const size_t NG = (size_t)k / group;
  uint32_t* out = (uint32_t*)codes_out;
  for (size_t s = 0; s < NS; ++s)
    for (size_t kt = 0; kt < KT; ++kt) {
      uint32_t* tile = out + (s * KT + kt) * 256;
      for (int L = 0; L < 64; ++L) {
        const int r = L & 15, g = L >> 4;
        const int8_t* wrow = w + (s * 16 + r) * (size_t)k + kt * 256;
        for (int qw = 0; qw < 4; ++qw) {
          uint32_t P = 0;
          for (int half = 0; half < 2; ++half) {  // m = 2qw + half
            const int m = 2 * qw + half;
            for (int d = 0; d < 4; ++d)
              for (int h = 0; h < 2; ++h) {
                const int kk = 32 * m + 8 * g + 2 * d + h;
                const int8_t v = wrow[kk];
                if (v < -1 || v > 1)
                  return fail(TERN_ERR_VALUE, "tern_pack: w[%zu][%zu]=%d not in {-1,0,1}",
                              s * 16 + r, kt * 256 + kk, (int)v);
                const int j = 4 * half + d;
                const int b = (h ? 30 : 14) - 2 * j;
                P |= encode(v) << b;
              }
          }
          tile[L * 4 + qw] = P;
        }
      }
      for (int r = 0; r < 16; ++r)
        for (size_t gi = 0; gi < GPT; ++gi)
          scales_out[((s * KT + kt) * 16 + r) * GPT + gi] =
              scales_f16[(s * 16 + r) * NG + kt * GPT + gi];
    }
  return ok();
}

tern_status tern_unpack(const void* codes, const uint16_t* scales_packed, int n, int k, int group,
                        int8_t* w_out, uint16_t* scales_out) {
  if (!codes || !w_out) return fail(TERN_ERR_NULL, "tern_unpack: NULL pointer");
  if ((scales_packed == nullptr) != (scales_out == nullptr))
    return fail(TERN_ERR_NULL, "tern_unpack: give both scale pointers or neither");
  tern_status st = check_shape(n, k, group);
  if (st != TERN_OK) return st;
  const size_t NS = (size_t)n / 16, KT = (size_t)k / 256, GPT = 256 / (size_t)group;
  const size_t NG = (size_t)k / group;
  const uint32_t* in = (const uint32_t*)codes;
  for (size_t s = 0; s < NS; ++s)
    for (size_t kt = 0; kt < KT; ++kt) {
      const uint32_t* tile = in + (s * KT + kt) * 256;
      for (int L = 0; L < 64; ++L) {
        const int r = L & 15, g = L >> 4;
        int8_t* wrow = w_out + (s * 16 + r) * (size_t)k + kt * 256;
        for (int qw = 0; qw < 4; ++qw) {
          const uint32_t P = tile[L * 4 + qw];
          for (int half = 0; half < 2; ++half) {
            const int m = 2 * qw + half;
            for (int d = 0; d < 4; ++d)
              for (int h = 0; h < 2; ++h) {
                const int j = 4 * half + d;
                const int b = (h ? 30 : 14) - 2 * j;
                const uint32_t c = (P >> b) & 3u;
                if (c == 2u)
                  return fail(TERN_ERR_VALUE, "tern_unpack: invalid code 10 in tile (%zu,%zu)", s,
                              kt);
                wrow[32 * m + 8 * g + 2 * d + h] = c == 0 ? 0 : (c == 1 ? 1 : -1);
              }
          }
        }
      }
      if (scales_out)
        for (int r = 0; r < 16; ++r)
          for (size_t gi = 0; gi < GPT; ++gi)
            scales_out[(s * 16 + r) * NG + kt * GPT + gi] =
                scales_packed[((s * KT + kt) * 16 + r) * GPT + gi];
    }
  return ok();
}

size_t tern_packed_code_bytes_t5(int n, int k) {
  if (n < 16 || n % 16 || k < 1024 || k % 1024 || k > kMaxK || n > kMaxN) return 0;
  return (size_t)n * (size_t)(k / 1024) * 208;
}

tern_status tern_pack_t5(const int8_t* w, const uint16_t* scales_f16, int n, int k, int group,
                         void* codes_out, uint16_t* scales_out) {
  if (!w || !scales_f16 || !codes_out || !scales_out)
    return fail(TERN_ERR_NULL, "tern_pack_t5: NULL pointer");
  tern_status st = check_shape(n, k, group);
  if (st != TERN_OK) return st;
  if (k % 1024 != 0) return fail(TERN_ERR_SHAPE, "layout t5: K=%d must be a multiple of 1024", k);
  const size_t NS = (size_t)n / 16, KQ = (size_t)k / 1024, KT = (size_t)k / 256;
  const size_t GPT = 256 / (size_t)group, NG = (size_t)k / group;
  for (size_t i = 0; i < (size_t)n * k; ++i)
    if (w[i] < -1 || w[i] > 1)
      return fail(TERN_ERR_VALUE, "tern_pack_t5: w[%zu][%zu]=%d not in {-1,0,1}", i / k, i % k, (int)w[i]);
  uint8_t* out = (uint8_t*)codes_out;
  // column of byte e of register R (R = 4q + i) of lane group g, in a k-tile
  auto col = [](int R, int e, int g) {
    const int q = R >> 2, i = R & 3;
    const int m = e == 0 ? 32 + 2 * i : e == 1 ? 2 * i : e == 2 ? 33 + 2 * i : 2 * i + 1;
    return 64 * q + 8 * g + m;
  };
  for (size_t s = 0; s < NS; ++s)
    for (size_t Q = 0; Q < KQ; ++Q) {
      uint8_t* blk = out + (s * KQ + Q) * 3328;
      for (int j = 0; j < 4; ++j)
        for (int L = 0; L < 64; ++L) {
          const int r = L & 15, g = L >> 4;
          const int8_t* wrow = w + (s * 16 + r) * (size_t)k + (Q * 4 + j) * 256;
          for (int word = 0; word < 3; ++word)
            for (int e = 0; e < 4; ++e) {
              int v = 0;  // trits t_0..t_4 of registers 5 word .. 5 word + 4, t_0 most significant
              for (int d = 0; d < 5; ++d) v = 3 * v + (wrow[col(5 * word + d, e, g)] + 1);
              blk[768 * j + 12 * L + 4 * word + e] = (uint8_t)((256 * v + 242) / 243);
            }
          int tail = 0;
          for (int e = 0; e < 4; ++e) tail |= (wrow[col(15, e, g)] + 1) << (2 * e);
          blk[3072 + 4 * L + j] = (uint8_t)tail;
        }
    }
  for (size_t s = 0; s < NS; ++s)
    for (size_t kt = 0; kt < KT; ++kt)
      for (int r = 0; r < 16; ++r)
        for (size_t gi = 0; gi < GPT; ++gi)
          scales_out[((s * KT + kt) * 16 + r) * GPT + gi] = scales_f16[(s * 16 + r) * NG + kt * GPT + gi];
  return ok();
}

tern_status tern_unpack_t5(const void* codes, const uint16_t* scales_packed, int n, int k, int group,
                           int8_t* w_out, uint16_t* scales_out) {
  if (!codes || !w_out) return fail(TERN_ERR_NULL, "tern_unpack_t5: NULL pointer");
  if ((scales_packed == nullptr) != (scales_out == nullptr))
    return fail(TERN_ERR_NULL, "tern_unpack_t5: give both scale pointers or neither");
  tern_status st = check_shape(n, k, group);
  if (st != TERN_OK) return st;
  if (k % 1024 != 0) return fail(TERN_ERR_SHAPE, "layout t5: K=%d must be a multiple of 1024", k);
  const size_t NS = (size_t)n / 16, KQ = (size_t)k / 1024, KT = (size_t)k / 256;
  const size_t GPT = 256 / (size_t)group, NG = (size_t)k / group;
  const uint8_t* in = (const uint8_t*)codes;
  auto col = [](int R, int e, int g) {
    const int q = R >> 2, i = R & 3;
    const int m = e == 0 ? 32 + 2 * i : e == 1 ? 2 * i : e == 2 ? 33 + 2 * i : 2 * i + 1;
    return 64 * q + 8 * g + m;
  };
  for (size_t s = 0; s < NS; ++s)
    for (size_t Q = 0; Q < KQ; ++Q) {
      const uint8_t* blk = in + (s * KQ + Q) * 3328;
      for (int j = 0; j < 4; ++j)
        for (int L = 0; L < 64; ++L) {
          const int r = L & 15, g = L >> 4;
          int8_t* wrow = w_out + (s * 16 + r) * (size_t)k + (Q * 4 + j) * 256;
          for (int word = 0; word < 3; ++word)
            for (int e = 0; e < 4; ++e) {
              const int b = blk[768 * j + 12 * L + 4 * word + e];
              int q = b;  // the kernel's decode: five times q = 3q, trit = q >> 8, q &= 255
              int v = 0;
              for (int d = 0; d < 5; ++d) {
                const int q3 = 3 * q;
                wrow[col(5 * word + d, e, g)] = (int8_t)((q3 >> 8) - 1);
                v = 3 * v + (q3 >> 8);
                q = q3 & 255;
              }
              if ((256 * v + 242) / 243 != b)
                return fail(TERN_ERR_VALUE, "tern_unpack_t5: byte 0x%02x is not a packed value", b);
            }
          const int tail = blk[3072 + 4 * L + j];
          for (int e = 0; e < 4; ++e) {
            const int t = (tail >> (2 * e)) & 3;
            if (t == 3) return fail(TERN_ERR_VALUE, "tern_unpack_t5: tail trit 3");
            wrow[col(15, e, g)] = (int8_t)(t - 1);
          }
        }
    }
  if (scales_out)
    for (size_t s = 0; s < NS; ++s)
      for (size_t kt = 0; kt < KT; ++kt)
        for (int r = 0; r < 16; ++r)
          for (size_t gi = 0; gi < GPT; ++gi)
            scales_out[(s * 16 + r) * NG + kt * GPT + gi] = scales_packed[((s * KT + kt) * 16 + r) * GPT + gi];
  return ok();
}

size_t tern_chain_counter_bytes(int count) { return count < 1 ? 0 : (size_t)(count + 1) * sizeof(int32_t); }

}  // extern "C"

namespace {

// Plans of a chain's items (the gemv's K split), validated: the shared part
// of tern_chain_table_bytes and tern_chain_build. The LDS layout of the
// kernel: two limb slots sized for the largest K, then the K-share sums.
struct ChainLayout {
  int rs = 0;          // bytes of one limb row (largest K + 64)
  int slot_bytes = 0;  // 3 limb rows and the k-tile exponents, 16-byte aligned
  int lds = 0;
};
tern_status chain_plan_items(const tern_chain_item* items, int count, std::vector<tern::ChainEntry>& t,
                             ChainLayout* lay) {
  if (!items) return fail(TERN_ERR_NULL, "chain: items is NULL");
  if (count < 1 || count > (1 << 20)) return fail(TERN_ERR_SHAPE, "chain: count=%d", count);
  const Config& c = config();
  if (!c.valid) return fail(TERN_ERR_CONFIG, "%s", c.error.c_str());
  t.assign((size_t)count, tern::ChainEntry{});
  const int group = items[0].W.group;
  int kmax = 0;
  for (int i = 0; i < count; ++i) {
    const tern_chain_item& it = items[i];
    tern_status st = check_weights(&it.W);
    if (st != TERN_OK) return fail(st, "chain item %d: %s", i, g_last_error.c_str());
    if (it.W.layout != TERN_LAYOUT_V1) return fail(TERN_ERR_LAYOUT, "chain item %d: layout v1 only", i);
    if (it.W.group != group) return fail(TERN_ERR_SHAPE, "chain item %d: group %d, item 0 has %d", i, it.W.group, group);
    if (!it.x || !it.y) return fail(TERN_ERR_NULL, "chain item %d: x or y is NULL", i);
    if (!aligned16(it.x) || !aligned16(it.y) || ((uintptr_t)it.y_bf16 & 3u))
      return fail(TERN_ERR_ALIGN, "chain item %d: x and y 16-byte, y_bf16 4-byte aligned", i);
    if (it.after < -1 || it.after >= i) return fail(TERN_ERR_VALUE, "chain item %d: after=%d", i, it.after);
    const tern::LimbPlan p = plan_limb(1, it.W.n, it.W.k);
    if (p.wk < 1 || p.wk > tern::kChainWaves)
      return fail(TERN_ERR_CONFIG, "chain item %d: %d K shares exceed %d waves", i, p.wk, tern::kChainWaves);
    kmax = std::max(kmax, it.W.k);
    tern::ChainEntry& e = t[(size_t)i];
    e.codes = it.W.codes;
    e.scales = it.W.scales;
    e.x = (const uint16_t*)it.x;
    e.y = it.y;
    e.y_bf16 = it.y_bf16;
    e.n = it.W.n;
    e.k = it.W.k;
    e.wk = p.wk;
    e.wn = p.wk == 1 ? 1 : tern::kChainWaves / p.wk;
    e.units = (it.W.n / 16 + e.wn - 1) / e.wn;
    e.after = it.after;
    e.signal = 0;
  }
  for (int i = 0; i < count; ++i)
    if (t[(size_t)i].after >= 0) t[(size_t)t[(size_t)i].after].signal = 1;
  lay->rs = kmax + 64;
  lay->slot_bytes = (3 * lay->rs + (kmax / 256) * 4 + 15) & ~15;
  lay->lds = 2 * lay->slot_bytes + 2 * tern::kChainWaves * 16 * 4;
  if (lay->lds > tern::kLimbMaxLdsResident)
    return fail(TERN_ERR_SHAPE, "chain: K=%d needs %d bytes of LDS (at most %d)", kmax, lay->lds,
                tern::kLimbMaxLdsResident);
  return TERN_OK;
}

// Work of a chain for P workgroups: the items are cut into stages at every
// item that depends on an item of the current stage; each stage's units (in item order) are dealt to the
// workgroups in contiguous runs of about equal cost, so a workgroup switches
// items (and makes new limbs) a few times per stage at most. Cost of a unit,
// in k-tiles a wave streams: wk = 1, one strip of KT k-tiles (dealt over the
// waves); wk > 1, every wave one share, the longest ceil(KT / wk), plus a
// barrier. Events per workgroup, in item order: its run of each item, and a
// signal after every item that a later one waits on.
std::vector<std::vector<std::array<int32_t, 4>>> chain_events(const std::vector<tern::ChainEntry>& t, int P) {
  std::vector<std::vector<std::array<int32_t, 4>>> ev((size_t)P);
  const int count = (int)t.size();
  for (int s0 = 0; s0 < count;) {
    // a stage runs on until an item depends on one inside it (items whose
    // dependency lies before the stage, like k and v beside q, join it)
    int s1 = s0 + 1;
    while (s1 < count && t[(size_t)s1].after < s0) ++s1;
    auto cost = [&](const tern::ChainEntry& e) {
      const int KT = e.k / 256;
      return e.wk == 1 ? (double)KT : (double)tern::kChainWaves * ((KT + e.wk - 1) / e.wk + 1);
    };
    double total = 0.0;
    for (int i = s0; i < s1; ++i) total += cost(t[(size_t)i]) * t[(size_t)i].units;
    const double per = total / P;
    double cum = 0.0;
    for (int i = s0; i < s1; ++i) {
      const tern::ChainEntry& e = t[(size_t)i];
      const double c = cost(e);
      int cur = -1, u0 = 0;
      for (int u = 0; u <= e.units; ++u) {
        const int w = u < e.units ? std::min(P - 1, (int)((cum + 0.5 * c) / per)) : -2;
        if (w != cur) {
          if (cur >= 0) ev[(size_t)cur].push_back({i, u0, u, 0});
          cur = w;
          u0 = u;
        }
        if (u < e.units) cum += c;
      }
      if (e.signal)
        for (int w = 0; w < P; ++w) ev[(size_t)w].push_back({i, 0, 0, 1});
    }
    s0 = s1;
  }
  return ev;
}

size_t chain_table_size(int count, size_t records) {
  return sizeof(int32_t) * 4 + (size_t)count * sizeof(tern::ChainEntry) + tern::kChainRecordOffsets * sizeof(int32_t) +
         records * 4 * sizeof(int32_t);
}

// Records of a chain at most, for any number of workgroups up to
// kChainMaxWorkgroups: every task, every unit end, every workgroup's switch
// to every item (a workgroup has at most one run of an item) and every
// signal, each of the last two for all 12 waves.
size_t chain_records_bound(const std::vector<tern::ChainEntry>& t) {
  const size_t P = tern::kChainMaxWorkgroups, W = tern::kChainWaves;
  size_t n = 0;
  for (const auto& e : t) {
    n += e.wk == 1 ? (size_t)e.units : (size_t)e.units * W;
    n += W * std::min(P, (size_t)e.units);
    if (e.signal) n += W * P;
  }
  return n;
}

// The events of each workgroup expanded into the record lists of its 12
// waves (the layout of tern_chain.hip): every wave gets the same switches,
// signals and unit ends in the same order; a wk = 1 run's strips go to the
// waves in turn, continuing from where the workgroup's previous run stopped.
std::vector<std::vector<std::array<int32_t, 4>>> chain_records(
    const std::vector<tern::ChainEntry>& t, const std::vector<std::vector<std::array<int32_t, 4>>>& ev) {
  const int W = tern::kChainWaves;
  std::vector<std::vector<std::array<int32_t, 4>>> rec(ev.size() * W);
  for (size_t b = 0; b < ev.size(); ++b) {
    auto* wr = &rec[b * W];
    int rot = 0, cur = -1, waited = -1;  // waited: the highest counter this workgroup has waited for
    for (const auto& e : ev[b]) {
      const int i = e[0];
      if (e[3] == 1) {
        for (int w = 0; w < W; ++w) wr[w].push_back({4 | (i << 4), 0, 0, 0});  // signal
        continue;
      }
      const tern::ChainEntry& c = t[(size_t)i];
      const int KT = c.k / 256, NS = c.n / 16;
      if (i != cur) {
        // item switch; y = 1: wait for counter `after` first (not needed
        // when the workgroup has already waited for it or a later one)
        const int wait = c.after > waited ? 1 : 0;
        if (wait) waited = c.after;
        for (int w = 0; w < W; ++w) wr[w].push_back({3 | (i << 4), wait, 0, 0});
        cur = i;
      }
      if (c.wk == 1) {
        for (int u = e[1]; u < e[2]; ++u) wr[(rot + u - e[1]) % W].push_back({0 | (i << 4), u, 0, KT << 16});
        rot = (rot + e[2] - e[1]) % W;
      } else {
        for (int u = e[1]; u < e[2]; ++u)
          for (int w = 0; w < W; ++w) {
            const int wn = w % c.wn, wk = w / c.wn, strip = u * c.wn + wn;
            if (wk < c.wk && strip < NS) {
              const int kt0 = (wk * KT) / c.wk, nkt = ((wk + 1) * KT) / c.wk - kt0;
              wr[w].push_back({1 | (i << 4), strip, u, kt0 | (nkt << 16)});
            } else {
              wr[w].push_back({2 | (i << 4), u, 0, 0});
            }
          }
      }
    }
  }
  return rec;
}

}  // namespace

extern "C" {

size_t tern_chain_table_bytes(const tern_chain_item* items, int count) {
  std::vector<tern::ChainEntry> t;
  ChainLayout lay;
  if (chain_plan_items(items, count, t, &lay) != TERN_OK) return 0;
  // the record count depends on the device's workgroups: a bound for the most
  return chain_table_size(count, chain_records_bound(t));
}

tern_status tern_chain_build(const tern_chain_item* items, int count, void* table, size_t table_bytes,
                             tern_chain_plan* plan) {
  if (!table || !plan) return fail(TERN_ERR_NULL, "tern_chain_build: NULL pointer");
  std::vector<tern::ChainEntry> t;
  ChainLayout lay;
  tern_status st = chain_plan_items(items, count, t, &lay);
  if (st != TERN_OK) return st;
  if (!aligned16(table)) return fail(TERN_ERR_ALIGN, "chain table must be 16-byte aligned");
  const int dev_max = tern::chain_max_workgroups(lay.lds);
  if (dev_max <= 0) return hip_fail(-dev_max, "chain occupancy query");
  int cus = 0;
  const int cerr = tern::device_cu_count(&cus);
  if (cerr) return hip_fail(cerr, "chain CU count");
  const int P = std::min(std::min(dev_max, cus), tern::kChainMaxWorkgroups);  // one workgroup per CU
  const auto rec = chain_records(t, chain_events(t, P));
  size_t nrec = 0;
  for (const auto& l : rec) nrec += l.size();
  const size_t need = chain_table_size(count, nrec);
  if (table_bytes < need) return fail(TERN_ERR_WORKSPACE, "chain table needs %zu bytes, got %zu", need, table_bytes);
  std::vector<char> blob(need, 0);
  int32_t* head = (int32_t*)blob.data();
  head[0] = lay.rs;
  head[1] = lay.slot_bytes;
  head[2] = count;
  head[3] = (int32_t)tern::kChainTableMagic;
  memcpy(blob.data() + 16, t.data(), t.size() * sizeof(tern::ChainEntry));
  int32_t* wv_begin = (int32_t*)(blob.data() + 16 + t.size() * sizeof(tern::ChainEntry));
  int32_t* recs = wv_begin + tern::kChainRecordOffsets;
  int32_t pos = 0;
  for (size_t v = 0; v < (size_t)tern::kChainRecordOffsets; ++v) {
    wv_begin[v] = pos;
    if (v < rec.size())
      for (const auto& e : rec[v]) {
        memcpy(recs + 4 * (size_t)pos, e.data(), sizeof(int32_t) * 4);
        ++pos;
      }
  }
  const int err = tern::copy_to_device(table, blob.data(), blob.size());
  if (err) return hip_fail(err, "chain table copy");
  plan->count = count;
  plan->group = items[0].W.group;
  plan->workgroups = P;
  plan->lds_bytes = lay.lds;
  plan->waits = 0;
  for (const auto& e : t) plan->waits |= e.after >= 0;
  return ok();
}

tern_status tern_linear_chain(const tern_chain_plan* plan, const void* table, void* counters,
                              size_t counter_bytes, int32_t* error_flag, int spin_limit, void* stream) {
  call_begin();
  if (!plan || !table || !counters || !error_flag) return fail(TERN_ERR_NULL, "tern_linear_chain: NULL pointer");
  if (plan->count < 1 || plan->workgroups < 1 || plan->workgroups > tern::kChainMaxWorkgroups ||
      (plan->group != 64 && plan->group != 128) || plan->lds_bytes < 0 || plan->lds_bytes > tern::kLimbMaxLdsResident)
    return fail(TERN_ERR_VALUE, "tern_linear_chain: plan not from tern_chain_build");
  if (counter_bytes < tern_chain_counter_bytes(plan->count))
    return fail(TERN_ERR_WORKSPACE, "chain counters need %zu bytes, got %zu", tern_chain_counter_bytes(plan->count),
                counter_bytes);
  if (spin_limit < 1) return fail(TERN_ERR_VALUE, "spin_limit=%d must be at least 1", spin_limit);
  if (!aligned16(table) || ((uintptr_t)counters & 3u) || ((uintptr_t)error_flag & 3u))
    return fail(TERN_ERR_ALIGN, "table 16-byte, counters and error_flag 4-byte aligned");
  const int err = tern::launch_chain(table, plan->count, plan->group, plan->workgroups, plan->lds_bytes,
                                     (int*)counters, (int*)error_flag, spin_limit, plan->waits != 0, stream);
  if (err) return hip_fail(err, "chain launch");
  return call_ok();
}

size_t tern_workspace_bytes(int T, int n, int k, int group, tern_rung rung) {
  if (check_shape(n, k, group) != TERN_OK) return (size_t)-1;
  tern_rung r;
  if (resolve(T, rung, &r) != TERN_OK) return (size_t)-1;
  return choose(T, n, k, group, r).workspace;
}

uint64_t tern_plan_kernels(int T, int n, int k, int group, uint32_t layout, tern_rung rung) {
  if (check_shape(n, k, group) != TERN_OK) return 0;
  if (layout != TERN_LAYOUT_V1 && layout != TERN_LAYOUT_T5) {
    fail(TERN_ERR_LAYOUT, "layout=0x%08x is neither TERN_LAYOUT_V1 nor TERN_LAYOUT_T5", layout);
    return 0;
  }
  if (layout == TERN_LAYOUT_T5 && k % 1024 != 0) {
    fail(TERN_ERR_SHAPE, "layout t5: K=%d must be a multiple of 1024", k);
    return 0;
  }
  tern_rung r;
  if (resolve(T, rung, &r) != TERN_OK) return 0;
  if (layout == TERN_LAYOUT_T5) {
    Choice c;
    return choose_t5(T, n, k, group, r, &c) == TERN_OK ? c.kernels : 0;
  }
  return choose(T, n, k, group, r).kernels;
}

int tern_resolve_rung(int T, tern_rung rung) {
  tern_rung r;
  const tern_status st = resolve(T, rung, &r);
  if (st != TERN_OK) return -(int)st;
  return (int)r;
}

tern_status tern_quant_act_s8(const void* x_bf16, int T, int k, int8_t* q, float* act_scale,
                              tern_q_layout layout, void* stream) {
  call_begin();
  if (!x_bf16 || !q || !act_scale) return fail(TERN_ERR_NULL, "tern_quant_act_s8: NULL pointer");
  if (T < 1 || T > kMaxTokens) return fail(TERN_ERR_SHAPE, "T=%d out of range", T);
  if (layout != TERN_Q_ROW_MAJOR && layout != TERN_Q_OPERAND_ORDER)
    return fail(TERN_ERR_VALUE, "unknown q layout %d", (int)layout);
  const int mult = layout == TERN_Q_OPERAND_ORDER ? 64 : 8;
  if (k < mult || k % mult != 0 || k > kMaxK)
    return fail(TERN_ERR_SHAPE, "K=%d must be a positive multiple of %d, at most %d", k, mult, kMaxK);
  if (!aligned16(x_bf16) || !aligned16(q))
    return fail(TERN_ERR_ALIGN, "x and q must be 16-byte aligned");
  int err = tern::launch_quant_s8((const uint16_t*)x_bf16, T, k, q, act_scale,
                                  layout == TERN_Q_OPERAND_ORDER, stream);
  if (err) return hip_fail(err, "quant_s8 launch");
  return call_ok();
}

tern_status tern_quant_act_s8_rot(const void* x_bf16, int T, int k, int8_t* q, float* act_scale,
                                  tern_q_layout layout, void* stream) {
  call_begin();
  if (!x_bf16 || !q || !act_scale) return fail(TERN_ERR_NULL, "tern_quant_act_s8_rot: NULL pointer");
  if (T < 1 || T > kMaxTokens) return fail(TERN_ERR_SHAPE, "T=%d out of range", T);
  if (layout != TERN_Q_ROW_MAJOR && layout != TERN_Q_OPERAND_ORDER)
    return fail(TERN_ERR_VALUE, "unknown q layout %d", (int)layout);
  if (k < 1024 || k % 1024 != 0 || k > tern::kRotMaxK)
    return fail(TERN_ERR_SHAPE, "K=%d must be a multiple of 1024 in [1024, %d]", k, tern::kRotMaxK);
  if (!aligned16(x_bf16) || !aligned16(q))
    return fail(TERN_ERR_ALIGN, "x and q must be 16-byte aligned");
  int err = tern::launch_quant_s8_rot((const uint16_t*)x_bf16, T, k, q, act_scale,
                                      layout == TERN_Q_OPERAND_ORDER, stream);
  if (err) return hip_fail(err, "quant_s8_rot launch");
  return call_ok();
}

tern_status tern_stream_read(const void* buf, size_t bytes, int depth, int waves_per_cu,
                             uint32_t* sink, void* stream) {
  call_begin();
  if (!buf || !sink) return fail(TERN_ERR_NULL, "tern_stream_read: NULL pointer");
  if (bytes < 1024 || bytes % 1024 != 0 || bytes / 1024 > 0x7fffffffu)
    return fail(TERN_ERR_SHAPE, "bytes=%zu must be a positive multiple of 1024 below 2 TiB", bytes);
  if (depth != 4 && depth != 8 && depth != 16)
    return fail(TERN_ERR_VALUE, "depth=%d must be 4, 8 or 16", depth);
  if (waves_per_cu < 1 || waves_per_cu > 32)
    return fail(TERN_ERR_VALUE, "waves_per_cu=%d must be in [1, 32]", waves_per_cu);
  if (!aligned16(buf) || ((uintptr_t)sink & 3u) != 0)
    return fail(TERN_ERR_ALIGN, "buf must be 16-byte and sink 4-byte aligned");
  const int err = tern::launch_stream_read(buf, bytes, depth, waves_per_cu, sink, stream);
  if (err) return hip_fail(err, "stream_read launch");
  return call_ok();
}

tern_status tern_linear(const void* x_bf16, int T, const tern_weights* W, float* y,
                        tern_rung rung, void* ws, size_t ws_bytes, void* stream) {
  call_begin();
  return linear_call(x_bf16, T, W, y, rung, ws, ws_bytes, stream, false);
}

tern_status tern_linear_noalloc(const void* x_bf16, int T, const tern_weights* W, float* y,
                                tern_rung rung, void* stream) {
  call_begin();
  return linear_call(x_bf16, T, W, y, rung, nullptr, tern::kNoallocScratchBytes, stream, true);
}

tern_status tern_linear_s8_q(const int8_t* q, const float* act_scale, int T,
                             const tern_weights* W, float* y, tern_q_layout layout, void* stream) {
  call_begin();
  if (!q || !act_scale || !y) return fail(TERN_ERR_NULL, "tern_linear_s8_q: NULL pointer");
  tern_status st = check_weights(W);
  if (st != TERN_OK) return st;
  if (T < 1 || T > kMaxTokens) return fail(TERN_ERR_SHAPE, "T=%d out of range", T);
  if (layout != TERN_Q_ROW_MAJOR && layout != TERN_Q_OPERAND_ORDER)
    return fail(TERN_ERR_VALUE, "unknown q layout %d", (int)layout);
  if (!aligned16(q) || !aligned16(y)) return fail(TERN_ERR_ALIGN, "q and y must be 16-byte aligned");
  const Config& c = config();
  if (!c.valid) return fail(TERN_ERR_CONFIG, "%s", c.error.c_str());
  tern::S8Args a{q,       act_scale, T,       W->k,    W->n, W->group, W->codes,
                 W->scales, y,       nullptr, layout == TERN_Q_OPERAND_ORDER};
  int err = tern::launch_s8(a, plan_s8(T, W->n, W->k, false), nullptr, stream);
  if (err) return hip_fail(err, "s8 launch");
  probe_hit(TERN_RUNG_S8, T, W->n, W->k, W->group);
  return call_ok();
}

tern_status tern_debug_s8_acc(const int8_t* q, int T, const tern_weights* W, int32_t* acc_out,
                              tern_q_layout layout, void* stream) {
  call_begin();
  if (!q || !acc_out) return fail(TERN_ERR_NULL, "tern_debug_s8_acc: NULL pointer");
  tern_status st = check_weights(W);
  if (st != TERN_OK) return st;
  if (T < 1 || T > kMaxTokens) return fail(TERN_ERR_SHAPE, "T=%d out of range", T);
  if (layout != TERN_Q_ROW_MAJOR && layout != TERN_Q_OPERAND_ORDER)
    return fail(TERN_ERR_VALUE, "unknown q layout %d", (int)layout);
  if (!aligned16(q)) return fail(TERN_ERR_ALIGN, "q must be 16-byte aligned");
  const Config& c = config();
  if (!c.valid) return fail(TERN_ERR_CONFIG, "%s", c.error.c_str());
  tern::S8Args a{q,       nullptr, T,      W->k, W->n, W->group, W->codes, W->scales,
                 nullptr, acc_out, layout == TERN_Q_OPERAND_ORDER};
  tern::S8Plan p = plan_s8(T, W->n, W->k, false);
  p.depth = 2;  // the export runs the double-buffered pipeline
  if (p.token_blocks * p.strips >= 16) p.strips = 2;  // and the 64 x 64 tile as 64 x 32 (registers)
  int err = tern::launch_s8(a, p, nullptr, stream);
  if (err) return hip_fail(err, "s8 debug launch");
  return call_ok();
}

void tern_probe_snapshot(uint64_t out[TERN_RUNG_COUNT]) {
  for (int i = 0; i < TERN_RUNG_COUNT; ++i) out[i] = g_probe[i].load(std::memory_order_relaxed);
}

void tern_probe_reset(void) {
  for (int i = 0; i < TERN_RUNG_COUNT; ++i) g_probe[i].store(0, std::memory_order_relaxed);
  for (int i = 0; i < TERN_KERNEL_COUNT; ++i) g_kprobe[i].store(0, std::memory_order_relaxed);
  g_last_rung.store(TERN_RUNG_AUTO, std::memory_order_relaxed);
}

void tern_kernel_probe_snapshot(uint64_t out[TERN_KERNEL_COUNT]) {
  for (int i = 0; i < TERN_KERNEL_COUNT; ++i) out[i] = g_kprobe[i].load(std::memory_order_relaxed);
}

uint64_t tern_last_kernels(void) { return t_last_kernels; }

const char* tern_kernel_name(tern_kernel kernel) {
  if ((int)kernel < 0 || (int)kernel >= TERN_KERNEL_COUNT) return "invalid";
  return kKernelNames[kernel];
}

tern_rung tern_last_rung(void) { return (tern_rung)g_last_rung.load(std::memory_order_relaxed); }

}  // extern "C"
