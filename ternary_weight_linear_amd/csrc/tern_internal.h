// tern_internal.h -- interface between the host ABI layer (tern_host.cpp) and
// the launchers of the gfx950 kernels (tern_*.hip). Not installed, not part
// of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/tern.h"

namespace tern {

// Kernel probe (tern_host.cpp): counts one launch of kernel `k` when `err`
// (a hipError_t value) is 0, i.e. the launch succeeded; returns `err`. Every
// launcher passes its hipGetLastError() through this at the launch site.
int kernel_launched(int err, tern_kernel k);

// Launch shape of the bf16-activation MFMA kernel (gemv / small_t / small_t_tiled).
struct SmallTPlan {
  int tokens_per_tile;  // 1 (gemv: one token per grid row) or 16
  int strips_per_wave;  // S: 16-row strips each wave streams (1, 2 or 4)
  int waves;            // W: waves per workgroup, each takes a contiguous K range (1..16)
  int token_tiles;      // grid.y
};

struct SmallTArgs {
  const uint16_t* x;  // bf16 [T][K]
  int T, K, N, G;
  const void* codes;
  const uint16_t* scales;
  float* y;  // [T][N]
};

// Launch shape of the s8 integer MFMA kernel for operand-order activations
// (tern_s8mma.hip), also used by the bf16 prefill kernel (tern_b16mma.hip):
// a wave tile of token_blocks x 16 tokens by strips x 16 outputs, (tb, s) in
// {(2,1), (3,1), (2,2), (2,4), (4,1), (4,2), (4,4)} (the bf16 prefill runs
// (4,4) as (4,2) and 3 blocks as 4). The kernel for row-major activations
// (tern_s8.hip) has one fixed shape.
struct S8Plan {
  int token_blocks;
  int strips;
  bool xcd_order;  // give each XCD a contiguous run of tiles (else plain block order)
  int k_parts;     // s8: K split over workgroups (> 1: fp32 partials in the workspace, then a reduce kernel)
  int depth;       // s8: k-tiles in flight, 2 or 4
};

struct S8Args {
  const int8_t* q;         // int8 [T][K]
  const float* act_scale;  // [T]
  int T, K, N, G;
  const void* codes;
  const uint16_t* scales;
  float* y;          // [T][N] (nullptr in debug-acc mode)
  int32_t* acc_out;  // [T][N][K/G] (debug-acc mode only)
  bool q_operand_order;  // q is in the s8 operand order (from launch_quant_s8(..., true, ...))
};

// Launch shape of the activation-tiled small-T kernel (tern_tile.hip).
struct TilePlan {
  int rows;             // activation rows staged per tile: 8 (T <= 8) or 16
  int strips_per_wave;  // S: 1, 2 or 4
  int waves;            // Ws: compute waves per workgroup (1..8), each owning S strips; plus a loader wave
  int depth;            // D: k-tiles of codes (per wave) and of activations in flight: 2, 4 or 8
  int strip_blocks;     // grid.x = ceil(NS / (Ws * S))
  int k_parts;          // grid.y = Pk: K split across workgroups (partials in the workspace)
  int token_tiles;      // grid.z = ceil(T / 16)
};

// Launch shape of the integer-limb decode kernel (tern_limb.hip), T <= 5.
struct LimbPlan {
  int strips_per_wave;  // S: 1, 2 or 4
  int wn;               // strip groups per workgroup (waves own different strips)
  int wk;               // K shares per workgroup (waves split the k-tiles); wn * wk <= 16
  int depth;            // k-tiles of codes in flight per wave: 2, 4 or 8
  bool token_lanes = false;  // T <= 4: lane group u holds token u (single-token epilogue)
  bool resident = false;     // limbs of the whole K in up to kLimbMaxLdsResident of LDS (one workgroup per CU)
  bool t5 = false;           // base-3 weights (layout t5): T = 1, one strip per wave, K % 1024 == 0
};
constexpr int kLimbMaxLds = 65536;
constexpr int kLimbMaxLdsResident = 160 * 1024;  // the resident small-T mode: all of a CU's LDS

// Launch shape of the small_t limb path (tern_limbtile.hip), T <= 8.
struct LimbTilePlan {
  int strips_per_wave;  // S: 1 or 2
  int waves;            // Ws: compute waves per workgroup (1..8); plus a loader wave
  int depth;            // D: k-tiles in flight, 2 or 4
  int strip_blocks;     // grid.x = ceil(NS / (Ws * S))
  bool fused;           // T <= 4: the loader wave makes the limbs (one launch, no workspace)
};

// Launch shape of the narrow-layer small-T kernel (tern_narrow.hip).
struct NarrowPlan {
  int rows;          // activation rows staged per k-tile: 4, 8 or 16 (>= T)
  int waves;         // W: waves per workgroup, one strip each: 8 or 16
  int kmax;          // k-tiles of codes requested up front per wave: 4, 8, 12 or 16 (>= ceil(KT / Pk))
  int strip_blocks;  // ceil(NS / W)
  int k_parts;       // Pk: K split over workgroups, partials added in the same launch
  int depth;         // k-tiles of codes in flight per wave: 4, or 0 (all kmax requested up front)
};

// All launchers return 0 on success or a hipError_t value.
int launch_small_t(const SmallTArgs& a, const SmallTPlan& p, void* stream);
// ws: tile_workspace_bytes(p, N) bytes of fp32 partials (k_parts > 1, added
// by a second kernel); may be NULL when that is 0.
int launch_tile(const SmallTArgs& a, const TilePlan& p, void* ws, void* stream);
size_t tile_workspace_bytes(const TilePlan& p, int N);
// T <= 5 tokens; needs limb_lds_bytes(T, K, G, p) <= kLimbMaxLds.
int launch_limb(const SmallTArgs& a, const LimbPlan& p, void* stream);
// T <= 8: limbs made by a prep kernel into ws (limbtile_workspace_bytes(T, K)
// bytes), then the contraction.
int launch_limbtile(const SmallTArgs& a, const LimbTilePlan& p, void* ws, void* stream);
size_t limbtile_workspace_bytes(int T, int K);
int limb_lds_bytes(int T, int K, int G, const LimbPlan& p);
// Largest waves-per-block the bf16 kernel accepts for this variant (LDS and
// register limits; 0 if none fits).
int small_t_max_waves(int tokens_per_tile, int strips, int K);
int small_t_lds_bytes(int tokens_per_tile, int strips, int waves, int K);
// operand_order: write q in the s8 kernel's operand order (K % 64 == 0)
// instead of row-major.
int launch_quant_s8(const uint16_t* x, int T, int K, int8_t* q, float* scale, bool operand_order,
                    void* stream);
// Rotated variant: 1024-wide blocks, K a multiple of 1024 up to kRotMaxK.
constexpr int kRotMaxK = 32768;
int launch_quant_s8_rot(const uint16_t* x, int T, int K, int8_t* q, float* scale, bool operand_order,
                        void* stream);
// ws: s8_partial_bytes(p, T, N) bytes of fp32 partials (k_parts > 1; operand
// order only), may be NULL when that is 0.
int launch_s8(const S8Args& a, const S8Plan& p, void* ws, void* stream);
size_t s8_partial_bytes(const S8Plan& p, int T, int N);
int launch_s8_operand_order(const S8Args& a, const S8Plan& p, void* ws, void* stream);
// part: narrow_partial_bytes(p, T, N) bytes; counters: strip_blocks ints,
// zero on entry, zero again when the launch completes (both unused when
// k_parts == 1).
int launch_narrow(const SmallTArgs& a, const NarrowPlan& p, void* part, int* counters, void* stream);
size_t narrow_partial_bytes(const NarrowPlan& p, int T, int N);
int narrow_lds_bytes(const NarrowPlan& p);
// bf16 prefill contraction (tern_b16mma.hip): the small_t_tiled rung above
// one 16-token tile; same tile plan as the s8 contraction.
int launch_b16_prefill(const SmallTArgs& a, const S8Plan& p, void* stream);

// Streaming-read ceiling probe (tern_probe.hip): one launch that reads
// `bytes` (a multiple of 1024) with `depth` (4, 8, 16) loads in flight per
// wave and about waves_per_cu waves per CU.
int launch_stream_read(const void* buf, size_t bytes, int depth, int waves_per_cu, uint32_t* sink,
                       void* stream);
const char* hip_error_string(int err);

// One projection of a decode chain (tern_chain.hip) as its kernel reads it:
// built on the host by tern_chain_build and copied to device memory once.
struct ChainEntry {
  const void* codes;       // layout v1
  const uint16_t* scales;  // re-laid fp16 scales
  const uint16_t* x;       // bf16 [K]
  float* y;                // fp32 [N]
  uint16_t* y_bf16;        // bf16 [N] or nullptr
  int32_t n, k;
  int32_t wn, wk;          // wk: the gemv's K shares; wn: strips per unit (12 / wk; 1 when wk = 1)
  int32_t units;           // wk > 1: ceil(N / 16 / wn) units; wk = 1: N / 16 strips
  int32_t after;           // -1, or j: read x once items 0..j have all finished
  int32_t signal;          // 1: a later item waits on this one (its workgroups count themselves done)
  int32_t pad[3];          // 80 bytes: what follows the entries stays 16-byte aligned
};
static_assert(sizeof(ChainEntry) == 80, "chain table layout");
constexpr int kChainWaves = 12;  // waves per workgroup of the chain kernel (one workgroup per CU)
constexpr int kChainMaxWorkgroups = 512;
constexpr unsigned kChainTableMagic = 0x4e484331u;  // "1CHN"
constexpr int kChainRecordOffsets = kChainMaxWorkgroups * kChainWaves + 4;
// Device table of a chain:
//   int4 header {row bytes of a limb row, bytes of an LDS limb slot, count, kChainTableMagic};
//   count ChainEntry;
//   kChainRecordOffsets ints: wave v = workgroup * kChainWaves + wave reads records
//   [wv_begin[v], wv_begin[v + 1]);
//   int4 records {type | item << 4, strip or unit, unit, kt0 | nkt << 16} (tern_chain.hip): every
//   wave of a workgroup holds the same item switches, signals and unit ends, in the same order, and
//   its own tasks among them.
// LDS of the kernel: two limb slots of slot_bytes (3 limb rows, then the
// k-tile exponents), then 2 x 12 x 16 floats of K-share sums.
// Launches the chain kernel: `workgroups` workgroups of kChainWaves waves
// (a cooperative launch when some item waits), `lds` bytes of dynamic LDS, group size 64 or 128 for
// every item. counters: count + 1 zeroed ints (left zeroed); error_flag: set
// to 1 by a wait that gives up after spin_limit polls, or when the table
// does not fit the launch.
int launch_chain(const void* table, int count, int group, int workgroups, int lds, int* counters, int* error_flag,
                 int spin_limit, bool cooperative, void* stream);
int chain_max_workgroups(int lds);  // co-resident workgroups of the chain kernel (negative: -hipError_t)
int device_cu_count(int* cus);      // compute units of the current device; returns a hipError_t value
int copy_to_device(void* dst, const void* src, size_t bytes);  // synchronous; returns a hipError_t value

// Static device scratch of tern_linear_noalloc (tern_noalloc.hip): its size,
// and the device address of the current device's copy (resolved with
// hipGetSymbolAddress on the first call per device). Returns a hipError_t value.
constexpr size_t kNoallocScratchBytes = (size_t)TERN_NOALLOC_SCRATCH_BYTES;
int noalloc_scratch(void** out);

}  // namespace tern
