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
// activation tile comes from: every compute wave of a workgroup owns
// different strips over the same k range, and each k-tile of activations is
// staged once per workgroup in LDS, so the activation traffic from L2 is one
// tile per workgroup instead of one per wave.
//
// Bytes in flight. The codes stream from HBM at about 2 us of latency, so a
// CU needs tens of KB of requests outstanding. Each compute wave keeps D
// k-tiles of its codes in flight in registers. The activation tiles are
// staged by one extra loader wave with direct buffer-to-LDS loads, D tiles
// ahead in a ring of D + 1 LDS buffers: the loader waits only for its own
// loads (the vector-memory counter retires loads in order, so a wave that
// staged activations and prefetched codes would have to wait for codes it
// does not need yet), and the compute waves only for their codes. One
// barrier per k-tile hands each tile over.
//
// K can also be split across Pk workgroups (TERN_TUNE_KPARTS; narrow layers
// now run tern_narrow.hip, which adds its parts inside the launch). Each
// workgroup writes fp32 partial sums to the workspace and a second, small
// kernel adds the Pk partials in ascending order (deterministic); the kernel
// boundary orders the two.
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
// operand read touches fall in different banks. The loader wave fills a tile
// with ROWS/2 direct loads of 64 lanes x 16 bytes: lane l of load c writes
// position 64c + l, i.e. row t = (64c + l) / 32, and fetches that row's
// global chunk (position ^ (t & 15)). Rows past the last token, and k-tiles
// past the last one (voffset beyond the resource), read as zeros.
template <int ROWS>
__device__ __forceinline__ void tile_stage_x(rsrc_t xrs, char* buf, int K, int kt, int lane, bool valid) {
  kt = __builtin_amdgcn_readfirstlane(kt);
#pragma unroll
  for (int c = 0; c < ROWS / 2; ++c) {
    const int p = 64 * c + lane;
    const int t = p >> 5;
    const int cl = (p & 31) ^ (t & 15);
    const int off = valid ? (t * K + cl * 8) * 2 : kOffPastEnd;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (__attribute__((address_space(3))) void*)(buf + 1024 * c),
                                             16, off, kt * 512, 0, 0);
  }
}

// The loader's side of a k-tile handoff: wait until at most N of its
// buffer-to-LDS loads are outstanding (vmcnt <= N; the loads retire in
// order), then the workgroup barrier. The barrier is issued without the
// workgroup fence of __syncthreads(): that fence would wait for every
// outstanding buffer-to-LDS load (vmcnt(0)) and so throw away the loader's
// lead. The "memory" clobber keeps the compiler from moving the next tile's
// loads above the barrier; the compute waves pass their own barriers through
// __syncthreads().
template <int N>
__device__ __forceinline__ void loader_handoff() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  asm volatile("s_barrier" ::: "memory");
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

// Grid: x = strip blocks (Ws*S strips), y = K parts (Pk), z = 16-token tiles.
// Block: Ws compute waves, wave w owning strips [sb*Ws*S + w*S, +S) over the
// block's K part, then the loader wave. Dynamic LDS: D + 1 activation tiles
// of ROWS*512 bytes.
template <int ROWS, int S, int GPT, int D>
__global__ void __launch_bounds__(576) tern_tile_kernel(
    const uint16_t* __restrict__ x, int T, int K, const u32x4* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int N, float* __restrict__ part) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TILE = ROWS * 512;
  constexpr int NB = D + 1;  // LDS tile ring
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Ws = (blockDim.x >> 6) - 1;  // compute waves; wave Ws is the loader
  const int NS = N >> 4, KT = K >> 8;
  const int sb = blockIdx.x, pk = blockIdx.y, tile = blockIdx.z;
  const int Pk = gridDim.y;
  const int kt0 = (pk * KT) / Pk;
  const int nkt = ((pk + 1) * KT) / Pk - kt0;
  const int t0 = tile * 16;

  if (wave == Ws) {
    // Loader: tiles 0..D-1, then per k-tile i the tile i + D into the buffer
    // of tile i - 1 (finished by every wave before the previous barrier),
    // and a wait until tile i + 1 has landed (D - 1 tiles may stay in flight).
    const rsrc_t xrs = make_rsrc(x + (size_t)t0 * K, (uint32_t)min(16, T - t0) * K * 2);
#pragma unroll
    for (int j = 0; j < D; ++j) tile_stage_x<ROWS>(xrs, smem + j * TILE, K, kt0 + j, lane, j < nkt);
    loader_handoff<(D - 1) * (ROWS / 2)>();
    for (int i = 0; i < nkt; ++i) {
      tile_stage_x<ROWS>(xrs, smem + ((i + D) % NB) * TILE, K, kt0 + i + D, lane, i + D < nkt);
      loader_handoff<(D - 1) * (ROWS / 2)>();
    }
    return;
  }

  const int strip0 = (sb * Ws + wave) * S;
  const int nstrips = min(S, NS - strip0);  // <= 0: the wave only keeps the barriers
  const rsrc_t crs = make_rsrc(codes + (size_t)max(min(strip0, NS - 1), 0) * KT * 64,
                               (uint32_t)max(nstrips, 0) * KT * 1024);
  const rsrc_t srs = make_rsrc(scales + (size_t)max(min(strip0, NS - 1), 0) * KT * 16 * GPT,
                               (uint32_t)max(nstrips, 0) * KT * 16 * GPT * 2);

  f32x4 total[S];
#pragma unroll
  for (int s = 0; s < S; ++s) total[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Code ring: stage j holds k-tile i + j; k-tile i + D - 1 is requested
  // before k-tile i is computed.
  TileStage<S, GPT> cb[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    tile_load_codes(cb[j], crs, srs, lane, KT, nstrips, kt0 + j, j < nkt);
  __syncthreads();

  int i = 0;
  for (; i + D <= nkt; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int ii = i + j;
      tile_load_codes(cb[(j + D - 1) % D], crs, srs, lane, KT, nstrips, kt0 + ii + D - 1,
                      ii + D - 1 < nkt);
      __builtin_amdgcn_sched_barrier(0);
      tile_compute<ROWS>(cb[j], total, smem + (ii % NB) * TILE, lane);
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j) {
    if (i + j < nkt) {  // uniform over the block
      const int ii = i + j;
      tile_compute<ROWS>(cb[j], total, smem + (ii % NB) * TILE, lane);
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
// order; four outputs per thread, token t = blockIdx.y. The parts are
// requested 8 at a time before they are added: they were just written on
// other XCDs, so each load is a full memory round trip, and a loop that
// waited for each in turn would pay Pk of them.
__global__ void __launch_bounds__(256) tern_tile_reduce_kernel(const float* __restrict__ part,
                                                              float* __restrict__ y, int N, int Pk) {
  const int n4 = N >> 2;
  const int c = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int t = (int)blockIdx.y;
  if (c >= n4) return;
  const f32x4* src = (const f32x4*)(part + ((size_t)(t >> 4) * Pk * 16 + (t & 15)) * N) + c;
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < Pk; p0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (p0 + j < Pk) v[j] = __builtin_nontemporal_load(src + (size_t)(p0 + j) * 16 * n4);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (p0 + j < Pk) sum += v[j];
  }
  ((f32x4*)(y + (size_t)t * N))[c] = sum * 0.5f;
}

template <int ROWS, int S, int GPT>
hipError_t launch_tile_g(const SmallTArgs& a, const TilePlan& p, float* part, hipStream_t st) {
  dim3 grid(p.strip_blocks, p.k_parts, p.token_tiles);
  dim3 block(64 * (p.waves + 1));
  const size_t lds = (size_t)(p.depth + 1) * ROWS * 512;
  // S * D <= 8: more code registers than that would not fit the 168 VGPRs a
  // 9-wave workgroup leaves each wave.
  switch (p.depth) {
#define TERN_TILE_LAUNCH(D)                                                                       \
  case D:                                                                                         \
    if constexpr (S * D <= 8)                                                                     \
      hipLaunchKernelGGL((tern_tile_kernel<ROWS, S, GPT, D>), grid, block, lds, st, a.x, a.T, a.K, \
                         (const u32x4*)a.codes, a.scales, a.y, a.N, part);                        \
    else                                                                                          \
      return hipErrorInvalidValue;                                                                \
    break;
    TERN_TILE_LAUNCH(2)
    TERN_TILE_LAUNCH(4)
    TERN_TILE_LAUNCH(8)
#undef TERN_TILE_LAUNCH
    default: return hipErrorInvalidValue;
  }
  return (hipError_t)kernel_launched((int)hipGetLastError(), TERN_KERNEL_SMALLT_TILE);
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
  if (p.depth != 2 && p.depth != 4 && p.depth != 8) return (int)hipErrorInvalidValue;
  if (p.k_parts > 1 && a.T > 65535) return (int)hipErrorInvalidValue;  // the reduce's grid.y
  float* part = p.k_parts > 1 ? (float*)ws : nullptr;
  hipError_t e = p.rows == 8 ? launch_tile_r<8>(a, p, part, st)
               : p.rows == 16 ? launch_tile_r<16>(a, p, part, st) : hipErrorInvalidValue;
  if (e != hipSuccess || p.k_parts == 1) return (int)e;
  hipLaunchKernelGGL(tern_tile_reduce_kernel, dim3((unsigned)((a.N / 4 + 255) / 256), (unsigned)a.T), dim3(256), 0,
                     st, (const float*)part, a.y, a.N, p.k_parts);
  return kernel_launched((int)hipGetLastError(), TERN_KERNEL_SMALLT_TILE_REDUCE);
}

}  // namespace tern
