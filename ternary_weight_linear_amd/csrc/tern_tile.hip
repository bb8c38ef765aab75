// tern_tile.hip -- small_t / small_t_tiled kernel (bf16 activations, up to 16
// tokens per tile) for gfx950.
//
// y[t][n] = sum_g s[n][g] * sum_{k in g} w[n][k] * x[t][k], w in {-1,0,+1},
// one fp16 scale per G weights along K ("NInfer sm_89 fork" article, section
// 9 item 2); T = 2..8 and 9..16 are the draft-verify rungs of the rung map
// ("NINFER ternary perf-tuning" notes, section 2).
//
// The activation tile (16 tokens x 256 k, bf16) is the A operand of
// v_mfma_f32_16x16x32_bf16 and the decoded codes of one 16-row strip its B
// operand, as in the single-token kernel. What differs is where the
// activation tile comes from: every wave of a workgroup owns different strips
// over the same k range, and the workgroup stages each k-tile of activations
// once in LDS (triple-buffered, one barrier per k-tile), so the activation
// traffic from L2 is one tile per workgroup instead of one per wave.
//
// Long K and narrow N (the down projection: 320 strips, 68 k-tiles) need more
// parallelism than the strips give, so K can also be split across Pk
// workgroups. Each writes fp32 partial sums to the workspace and a second,
// small kernel adds the Pk partials in ascending order (deterministic). The
// kernel boundary orders the two; a ticket-counter handoff inside one kernel
// would need a device-scope release per workgroup, i.e. an L2 writeback each,
// which on this part costs far more than the second launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

template <int S, int GPT>
struct TileStage {
  u32x4 P[S];
  uint32_t sw[S][GPT / 2];  // fp16 scale pairs of row (lane & 15)
};

template <int S, int GPT>
__device__ __forceinline__ void tile_load_codes(TileStage<S, GPT>& b, rsrc_t crs, rsrc_t srs,
                                                int lane, int KT, int nstrips, int kt, bool valid) {
  kt = __builtin_amdgcn_readfirstlane(min(max(kt, 0), KT - 1));
  const int cv = valid ? lane * 16 : kOffPastEnd;
  const int sv = valid ? (lane & 15) * GPT * 2 : kOffPastEnd;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int se = max(min(s, nstrips - 1), 0);  // absent strips re-read a present one (never stored)
    b.P[s] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, cv, (se * KT + kt) * 1024, kAuxNontemporal));
    const int soff = (se * KT + kt) * 16 * GPT * 2;
    if (GPT == 2) {
      b.sw[s][0] = __builtin_amdgcn_raw_buffer_load_b32(srs, sv, soff, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(srs, sv, soff, 0);
      b.sw[s][0] = v[0];
      b.sw[s][GPT / 2 - 1] = v[1];
    }
  }
}

// Activation tile in LDS: ROWS x 32 chunks of 16 bytes (8 bf16); chunk c of
// row t sits at position t*32 + (c ^ (t & 15)), so the 16 rows that an MFMA
// operand read touches fall in different banks. Loaded in 64-lane steps:
// step c covers positions [64c, 64c + 64); wave w of Ws issues steps
// w, w + Ws, ... (NXI of them) into registers, stored to LDS two k-tiles
// later.
template <int NXI>
struct XRegs {
  u32x4 v[NXI];
};

template <int ROWS, int NXI>
__device__ __forceinline__ void tile_load_x(XRegs<NXI>& r, rsrc_t xrs, int K, int kt, int wave,
                                            int Ws, int lane, bool valid) {
  kt = __builtin_amdgcn_readfirstlane(min(max(kt, 0), (K >> 8) - 1));
#pragma unroll
  for (int j = 0; j < NXI; ++j) {
    const int c = wave + Ws * j;
    const int p = 64 * c + lane;
    const int t = p >> 5;
    const int cl = (p & 31) ^ (t & 15);
    const int off = valid && c < ROWS / 2 ? (t * K + cl * 8) * 2 : kOffPastEnd;
    r.v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, kt * 512, 0));
  }
}

template <int ROWS, int NXI>
__device__ __forceinline__ void tile_store_x(const XRegs<NXI>& r, char* buf, int wave, int Ws,
                                             int lane) {
#pragma unroll
  for (int j = 0; j < NXI; ++j) {
    const int c = wave + Ws * j;
    if (c < ROWS / 2) *(u32x4*)(buf + (64 * c + lane) * 16) = r.v[j];
  }
}

// One k-tile: A fragments from the LDS tile, S strips x 8 MFMAs, fp32 scale
// epilogue per group (accumulator i of lane l is C[4(l>>4)+i][l&15]).
template <int ROWS, int S, int GPT>
__device__ __forceinline__ void tile_compute(const TileStage<S, GPT>& b, f32x4 (&total)[S],
                                             const char* buf, int lane) {
  constexpr int MPG = 8 / GPT;
  const int t = ROWS == 16 ? (lane & 15) : (lane & 7);  // rows >= ROWS only feed discarded outputs
  const int g = lane >> 4;
  const char* row = buf + t * 512;
  bf16x8 xa[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) xa[m] = *(const bf16x8*)(row + (((4 * m + g) ^ (t & 15)) << 4));
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint4 P = uint4{b.P[s].x, b.P[s].y, b.P[s].z, b.P[s].w};
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mm = 0; mm < MPG; ++mm) {
        const int m = gi * MPG + mm;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m], weights_operand(P, m), acc, 0, 0, 0);
      }
      const uint32_t spair = b.sw[s][gi >> 1];
      const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
      total[s][0] = __builtin_fmaf(sc, acc[0], total[s][0]);
      total[s][1] = __builtin_fmaf(sc, acc[1], total[s][1]);
      total[s][2] = __builtin_fmaf(sc, acc[2], total[s][2]);
      total[s][3] = __builtin_fmaf(sc, acc[3], total[s][3]);
    }
  }
}

constexpr int kTileDepth = 2;  // code stages in flight per wave (even: the x ring has 2 slots)

// Grid: x = strip blocks (Ws*S strips), y = K parts (Pk), z = 16-token tiles.
// Block: Ws waves, wave w owns strips [sb*Ws*S + w*S, +S) over the block's K
// part. Dynamic LDS: 3 activation tiles of ROWS*512 bytes.
template <int ROWS, int S, int GPT, int NXI>
__global__ void __launch_bounds__(512) tern_tile_kernel(
    const uint16_t* __restrict__ x, int T, int K, const u32x4* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int N, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TILE = ROWS * 512;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Ws = blockDim.x >> 6;
  const int NS = N >> 4, KT = K >> 8;
  const int sb = blockIdx.x, pk = blockIdx.y, tile = blockIdx.z;
  const int Pk = gridDim.y;
  const int kt0 = (pk * KT) / Pk;
  const int nkt = ((pk + 1) * KT) / Pk - kt0;
  const int strip0 = (sb * Ws + wave) * S;
  const int nstrips = min(S, NS - strip0);  // <= 0: this wave only helps stage activations
  const int t0 = tile * 16;

  const rsrc_t crs = make_rsrc(codes + (size_t)max(min(strip0, NS - 1), 0) * KT * 64,
                               (uint32_t)max(nstrips, 0) * KT * 1024);
  const rsrc_t srs = make_rsrc(scales + (size_t)max(min(strip0, NS - 1), 0) * KT * 16 * GPT,
                               (uint32_t)max(nstrips, 0) * KT * 16 * GPT * 2);
  const rsrc_t xrs = make_rsrc(x + (size_t)t0 * K, (uint32_t)min(16, T - t0) * K * 2);

  f32x4 total[S];
#pragma unroll
  for (int s = 0; s < S; ++s) total[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prologue: activation tile 0 into LDS buffer 0, tiles 1 and 2 in registers,
  // the first kTileDepth - 1 code stages in flight.
  XRegs<NXI> xr[2];
  TileStage<S, GPT> cb[kTileDepth];
  tile_load_x<ROWS, NXI>(xr[0], xrs, K, kt0, wave, Ws, lane, 0 < nkt);
#pragma unroll
  for (int j = 0; j < kTileDepth - 1; ++j)
    tile_load_codes(cb[j], crs, srs, lane, KT, nstrips, kt0 + j, j < nkt);
  tile_load_x<ROWS, NXI>(xr[1], xrs, K, kt0 + 1, wave, Ws, lane, 1 < nkt);
  tile_store_x<ROWS, NXI>(xr[0], smem, wave, Ws, lane);
  tile_load_x<ROWS, NXI>(xr[0], xrs, K, kt0 + 2, wave, Ws, lane, 2 < nkt);
  __syncthreads();

  // Iteration i: store activation tile i+1 (registers -> LDS), load tile
  // i+3 and code stage i+kTileDepth-1, compute k-tile i, barrier. Tile i was
  // stored before the previous barrier; the buffer written here last held
  // tile i-2, which every wave finished before that barrier.
  int i = 0;
  for (; i + kTileDepth <= nkt; i += kTileDepth) {
#pragma unroll
    for (int j = 0; j < kTileDepth; ++j) {
      const int ii = i + j;
      tile_store_x<ROWS, NXI>(xr[(j + 1) & 1], smem + ((ii + 1) % 3) * TILE, wave, Ws, lane);
      tile_load_x<ROWS, NXI>(xr[(j + 1) & 1], xrs, K, kt0 + ii + 3, wave, Ws, lane, ii + 3 < nkt);
      tile_load_codes(cb[(j + kTileDepth - 1) % kTileDepth], crs, srs, lane, KT, nstrips,
                      kt0 + ii + kTileDepth - 1, ii + kTileDepth - 1 < nkt);
      __builtin_amdgcn_sched_barrier(0);
      tile_compute<ROWS>(cb[j], total, smem + (ii % 3) * TILE, lane);
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < kTileDepth - 1; ++j) {
    if (i + j < nkt) {  // uniform over the block
      const int ii = i + j;
      tile_store_x<ROWS, NXI>(xr[(j + 1) & 1], smem + ((ii + 1) % 3) * TILE, wave, Ws, lane);
      tile_compute<ROWS>(cb[j], total, smem + (ii % 3) * TILE, lane);
      __syncthreads();
    }
  }

  // Outputs of lane l: token t0 + 4(l>>4) + i, row (l & 15) of each strip.
  const int tq = 4 * (lane >> 4), nl = lane & 15;
  if (Pk == 1) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s >= nstrips) break;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t0 + tq + e < T) y[(size_t)(t0 + tq + e) * N + (strip0 + s) * 16 + nl] = 0.5f * total[s][e];
    }
    return;
  }
  // Split K: fp32 partials [tile][pk][16][N], added by tern_tile_reduce_kernel.
  float* mine = part + ((size_t)tile * Pk + pk) * 16 * N;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (s >= nstrips) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) mine[(size_t)(tq + e) * N + (strip0 + s) * 16 + nl] = total[s][e];
  }
}

// y[t][n] = 0.5 * sum_{p < Pk} part[t / 16][p][t % 16][n], parts in ascending
// order; four outputs per thread.
__global__ void __launch_bounds__(256) tern_tile_reduce_kernel(const float* __restrict__ part,
                                                              float* __restrict__ y, int T, int N,
                                                              int Pk) {
  const int n4 = N >> 2;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T * n4) return;
  const int t = (int)(i / n4), c = (int)(i % n4);
  const f32x4* src = (const f32x4*)(part + ((size_t)(t >> 4) * Pk * 16 + (t & 15)) * N) + c;
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < Pk; ++p) sum += __builtin_nontemporal_load(src + (size_t)p * 16 * n4);
  ((f32x4*)(y + (size_t)t * N))[c] = sum * 0.5f;
}

// Load steps per wave for one activation tile (ROWS/2 steps of 64 lanes over
// Ws waves), rounded up to a power of two.
int tile_load_steps(int rows, int waves) {
  const int n = (rows / 2 + waves - 1) / waves;
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8;
}

template <int ROWS, int S, int GPT>
hipError_t launch_tile_g(const SmallTArgs& a, const TilePlan& p, float* part, hipStream_t st) {
  dim3 grid(p.strip_blocks, p.k_parts, p.token_tiles);
  dim3 block(64 * p.waves);
  const size_t lds = (size_t)3 * ROWS * 512;
#define TERN_TILE_LAUNCH(NX)                                                                   \
  hipLaunchKernelGGL((tern_tile_kernel<ROWS, S, GPT, NX>), grid, block, lds, st, a.x, a.T, a.K, \
                     (const u32x4*)a.codes, a.scales, a.y, a.N, part)
  switch (tile_load_steps(ROWS, p.waves)) {
    case 1: TERN_TILE_LAUNCH(1); break;
    case 2: TERN_TILE_LAUNCH(2); break;
    case 4: TERN_TILE_LAUNCH(4); break;
    default: return hipErrorInvalidValue;
  }
#undef TERN_TILE_LAUNCH
  return hipGetLastError();
}

template <int ROWS, int S>
hipError_t launch_tile_s(const SmallTArgs& a, const TilePlan& p, float* part, hipStream_t st) {
  return a.G == 128 ? launch_tile_g<ROWS, S, 2>(a, p, part, st)
                    : launch_tile_g<ROWS, S, 4>(a, p, part, st);
}

template <int ROWS>
hipError_t launch_tile_r(const SmallTArgs& a, const TilePlan& p, float* part, hipStream_t st) {
  switch (p.strips_per_wave) {
    case 1: return launch_tile_s<ROWS, 1>(a, p, part, st);
    case 2: return launch_tile_s<ROWS, 2>(a, p, part, st);
    case 4: return launch_tile_s<ROWS, 4>(a, p, part, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t tile_workspace_bytes(const TilePlan& p, int N) {
  if (p.k_parts <= 1) return 0;
  return (size_t)p.token_tiles * p.k_parts * 16 * N * sizeof(float);
}

int launch_tile(const SmallTArgs& a, const TilePlan& p, void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (p.waves < 1 || p.waves > 8 || p.k_parts < 1 || p.token_tiles < 1 || p.strip_blocks < 1)
    return (int)hipErrorInvalidValue;
  if (tile_load_steps(p.rows, p.waves) > 4) return (int)hipErrorInvalidValue;
  float* part = p.k_parts > 1 ? (float*)ws : nullptr;
  hipError_t e = p.rows == 8 ? launch_tile_r<8>(a, p, part, st)
               : p.rows == 16 ? launch_tile_r<16>(a, p, part, st) : hipErrorInvalidValue;
  if (e != hipSuccess || p.k_parts == 1) return (int)e;
  const long n = (long)a.T * (a.N / 4);
  hipLaunchKernelGGL(tern_tile_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const float*)part, a.y, a.T, a.N, p.k_parts);
  return (int)hipGetLastError();
}

}  // namespace tern
