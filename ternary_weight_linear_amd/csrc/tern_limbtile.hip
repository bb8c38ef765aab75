// tern_limbtile.hip -- small_t rung (T = 2..8) on the integer matrix cores:
// the bf16 activations as int8 limbs, as in the gemv kernel (tern_limb.hip),
// made k-tile by k-tile by the loader wave of the contraction
// (tern_limbfuse_kernel, T <= 4) or once per call by a small kernel
// (tern_limb_prep_kernel + tern_limbtile_kernel).
//
// y[t][n] = sum_g s[n][g] * sum_{k in g} w[n][k] * x[t][k], w in {-1,0,+1},
// one fp16 scale per G weights along K ("NInfer sm_89 fork" article, section
// 9 item 2); T = 2..8 is the draft-verify rung of the rung map ("NINFER
// ternary perf-tuning" notes, section 2).
//
// Why: on bf16 operands the decode of the 2-bit codes costs 15 vector-ALU
// instructions per 32 weights and lane, which bounds the bf16 small-T kernels
// (tern_tile.hip); the int8 decode costs 7 per 64. The activations then enter
// the integer MFMA as limbs: per token and 256-wide k-tile, with 2^E <=
// max|x| < 2^(E+1) and d = E - 21, v = rne(x * 2^-d) = l0 + 256 l1 + 65536 l2
// (tern_device.h), exact for every activation within 2^14 of the tile
// maximum. Made up front inside the contraction they would cost every
// workgroup the whole activation row before its first k-tile; the fused
// kernel makes each k-tile's limbs in its loader wave just ahead of use, the
// two-kernel path has tern_limb_prep_kernel make them once for the
// contraction to read like any other operand.
//
// Operand layout: row block b (16 rows) holds tokens 4b..4b+3, token 4b + u
// in rows 4u (l0), 4u + 1 (l1), 4u + 2 (l2), row 4u + 3 zero. An MFMA
// accumulator row 4g + e then lives in lane group g, element e: every lane
// holds the three limbs of one token in its own registers and combines them
// without crossing lanes, 65536 a2 + (256 a1 + a0) with the bracket exact in
// int32. Inside each row the bytes are in the s8 operand order (byte
// 16g + 4i + e of a 64-byte block holds k = 8g + m(i, e), the order
// weights_operand_i8 gives the codes).
//
// The contraction is the activation-tiled kernel's structure (tern_tile.hip):
// a loader wave stages each k-tile of limb rows (RB x 16 rows x 256 bytes) in
// LDS with buffer-to-LDS loads, D tiles ahead, and the compute waves keep D
// k-tiles of codes in flight and meet it at one barrier per k-tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

// One thread per 16-element chunk j of token slot t (chunk j covers natural
// k = 64(j>>2) + 8(j&3) + 0..7 and + 32; the 16 chunks of a k-tile are one DPP
// row, KC16 = K/16 being a multiple of 16). Slots past T write zero rows and
// exponent 0, so every byte the contraction reads is defined.
__global__ void __launch_bounds__(256) tern_limb_prep_kernel(const uint16_t* __restrict__ x, int T, int K,
                                                            int slots, int8_t* __restrict__ limbs,
                                                            int* __restrict__ dsh) {
  const int KC16 = K >> 4, KT = K >> 8;
  const int c = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (c >= slots * KC16) return;  // whole DPP rows: slots * KC16 is a multiple of 16
  const int t = c / KC16, j = c - t * KC16;
  const int rb = t >> 2, u = t & 3;
  int8_t* row = limbs + ((size_t)rb * 16 + 4 * u) * K + 16 * j;
  u32x4 out0 = u32x4{0, 0, 0, 0}, out1 = out0, out2 = out0;
  int d = 0;
  if (t < T) {
    const uint16_t* src = x + (size_t)t * K + 64 * (j >> 2) + 8 * (j & 3);
    const u32x4 lo = *(const u32x4*)src;
    const u32x4 hi = *(const u32x4*)(src + 32);
    d = limb_shift(row16_max_u32(absmax16(lo, hi)));
    limb_chunk(lo, hi, d, out0, out1, out2);
  }
  *(u32x4*)row = out0;
  *(u32x4*)(row + K) = out1;
  *(u32x4*)(row + 2 * K) = out2;
  *(u32x4*)(row + 3 * K) = u32x4{0, 0, 0, 0};
  // 2^(d - 6) undoes the fixed point and the 64x code decode
  if ((j & 15) == 0) dsh[t * KT + (j >> 4)] = t < T ? d - 6 : 0;
}

template <int S, int GPT, int RB>
struct LimbTileStage {
  u32x4 P[S];
  uint32_t sw[S][GPT / 2];  // fp16 scale pairs of row (lane & 15)
  int dsh[RB];              // 2^dsh of this lane's token in each row block
};

// The loader's handoff (as in tern_tile.hip): wait for all but N of its own
// buffer-to-LDS loads, then a barrier without the workgroup fence.
template <int N>
__device__ __forceinline__ void limbtile_handoff() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  asm volatile("s_barrier" ::: "memory");
}

// Grid: x = strip blocks (Ws*S strips). Block: Ws compute waves (wave w owns
// strips [sb*Ws*S + w*S, +S) over all of K), then the loader wave. Dynamic
// LDS: D + 1 limb tiles of RB*16 rows x 256 bytes; 16-byte chunk q of row r
// at position r*16 + (q ^ (r & 15)).
template <int RB, int S, int GPT, int D>
__global__ void __launch_bounds__(576) tern_limbtile_kernel(
    const int8_t* __restrict__ limbs, const int* __restrict__ dsh_g, int T, int K,
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales, float* __restrict__ y, int N) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TILE = RB * 16 * 256;
  constexpr int NB = D + 1;
  constexpr int LOADS = RB * 4;  // 1 KiB loads per tile
  constexpr int KBPG = 4 / GPT;  // 64-wide k-blocks per scale group
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Ws = (blockDim.x >> 6) - 1;
  const int NS = N >> 4, KT = K >> 8;

  if (wave == Ws) {
    // Loader: tiles 0..D-1, then per k-tile i the tile i + D into the buffer
    // of tile i - 1, and a wait until tile i + 1 has landed.
    const rsrc_t lrs = make_rsrc(limbs, (uint32_t)RB * 16 * K);
    auto stage = [&](int kt, char* buf) {
      kt = __builtin_amdgcn_readfirstlane(min(kt, KT - 1));
#pragma unroll
      for (int c = 0; c < LOADS; ++c) {
        const int p = 64 * c + lane;
        const int r = p >> 4;
        const int q = (p & 15) ^ (r & 15);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)(buf + 1024 * c),
                                                 16, r * K + q * 16, kt * 256, 0, 0);
      }
    };
#pragma unroll
    for (int j = 0; j < D; ++j) stage(j, smem + j * TILE);
    limbtile_handoff<(D - 1) * LOADS>();
    for (int i = 0; i < KT; ++i) {
      stage(i + D, smem + ((i + D) % NB) * TILE);
      limbtile_handoff<(D - 1) * LOADS>();
    }
    return;
  }

  const int r = lane & 15, g = lane >> 4;
  const int strip0 = (blockIdx.x * Ws + wave) * S;
  const int nstrips = min(S, NS - strip0);  // <= 0: the wave only keeps the barriers
  const rsrc_t crs = make_rsrc(codes + (size_t)max(min(strip0, NS - 1), 0) * KT * 64,
                               (uint32_t)max(nstrips, 0) * KT * 1024);
  const rsrc_t srs = make_rsrc(scales + (size_t)max(min(strip0, NS - 1), 0) * KT * 16 * GPT,
                               (uint32_t)max(nstrips, 0) * KT * 16 * GPT * 2);
  const rsrc_t drs = make_rsrc(dsh_g, (uint32_t)RB * 4 * KT * 4);

  auto load = [&](LimbTileStage<S, GPT, RB>& b, int kt) {
    kt = __builtin_amdgcn_readfirstlane(min(kt, KT - 1));
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int se = max(min(s, nstrips - 1), 0);  // absent strips re-read a present one (never stored)
      b.P[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, lane * 16, (se * KT + kt) * 1024, kAuxNontemporal));
      const int soff = (se * KT + kt) * 16 * GPT * 2;
      if (GPT == 2) {
        b.sw[s][0] = __builtin_amdgcn_raw_buffer_load_b32(srs, r * GPT * 2, soff, 0);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(srs, r * GPT * 2, soff, 0);
        b.sw[s][0] = v[0];
        b.sw[s][1] = v[1];
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      b.dsh[rb] = (int)__builtin_amdgcn_raw_buffer_load_b32(drs, ((rb * 4 + g) * KT) * 4, kt * 4, 0);
  };

  float total[S][RB];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) total[s][rb] = 0.f;

  // One k-tile: per group the A fragments of its k-blocks (shared by the
  // strips), per strip and row block the MFMA chain, the limb combination
  // and the scale; 2^dsh once per k-tile.
  auto compute = [&](const LimbTileStage<S, GPT, RB>& b, const char* buf) {
    float part[S][RB];
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      i32x4 af[KBPG][RB];
#pragma unroll
      for (int kk = 0; kk < KBPG; ++kk)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int q = 4 * (gi * KBPG + kk) + g;
          af[kk][rb] = *(const i32x4*)(buf + ((rb * 16 + r) * 16 + (q ^ r)) * 16);
        }
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint32_t spair = b.sw[s][gi >> 1];
        const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
        i32x4 acc[RB];
#pragma unroll
        for (int kk = 0; kk < KBPG; ++kk) {
          const i32x4 bf = weights_operand_i8(b.P[s][gi * KBPG + kk]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[kk][rb], bf,
                                                            kk == 0 ? i32x4{0, 0, 0, 0} : acc[rb], 0, 0, 0);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int low = (int)(((uint32_t)acc[rb][1] << 8) + (uint32_t)acc[rb][0]);  // 256 a1 + a0
          const float v = __builtin_fmaf(65536.0f, (float)acc[rb][2], (float)low);
          part[s][rb] = gi == 0 ? sc * v : __builtin_fmaf(sc, v, part[s][rb]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) total[s][rb] += __builtin_ldexpf(part[s][rb], b.dsh[rb]);
  };

  LimbTileStage<S, GPT, RB> cb[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j) load(cb[j], j);
  __syncthreads();
  int i = 0;
  for (; i + D <= KT; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int ii = i + j;
      load(cb[(j + D - 1) % D], ii + D - 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(cb[j], smem + (ii % NB) * TILE);
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j) {
    if (i + j < KT) {  // uniform over the block
      compute(cb[j], smem + ((i + j) % NB) * TILE);
      __syncthreads();
    }
  }

  // Lane (r, g): output row r of each strip for token 4rb + g.
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (s >= nstrips) break;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int t = 4 * rb + g;
      if (t < T) y[(size_t)t * N + (strip0 + s) * 16 + r] = total[s][rb];
    }
  }
}

// Fused variant for T <= 4 (one row block): the loader wave makes the limbs
// itself, k-tile by k-tile, so the call is one launch. Lane (u, j) of the
// loader holds chunk j of token u's k-tile (D k-tiles of x in flight in its
// registers), takes the tile exponent over its 16-lane DPP row and writes its
// three limb chunks and, at j = 0, 2^(d - 6) as an exponent into the LDS stage;
// two stages alternate. Rows of absent tokens (u >= T) and rows 4u + 3 are
// never written: they only feed accumulators that are not stored.
constexpr int kFuseTile = 16 * 256;        // limb rows of one k-tile
constexpr int kFuseStage = kFuseTile + 16;  // + 4 ints of exponent shifts

template <int S, int GPT, int D>
__global__ void __launch_bounds__(576) tern_limbfuse_kernel(
    const uint16_t* __restrict__ x, int T, int K, const u32x4* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int N) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kFuseStage];
  constexpr int KBPG = 4 / GPT;  // 64-wide k-blocks per scale group
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Ws = (blockDim.x >> 6) - 1;
  const int NS = N >> 4, KT = K >> 8;

  if (wave == Ws) {
    const int u = lane >> 4, j = lane & 15;
    const bool tok = u < T;
    const rsrc_t xrs = make_rsrc(x, (uint32_t)T * K * 2);
    // chunk j of a k-tile: k = 64 (j >> 2) + 8 (j & 3) + 0..7 and + 32
    const int xoff = tok ? (u * K + 64 * (j >> 2) + 8 * (j & 3)) * 2 : kOffPastEnd;
    u32x4 xl[D], xh[D];
    auto fetch = [&](int slot, int kt) {
      kt = __builtin_amdgcn_readfirstlane(min(kt, KT - 1));
      xl[slot] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff, kt * 512, 0));
      xh[slot] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff + 64, kt * 512, 0));
    };
    // Lanes of absent tokens skip the work: a DPP row (16 lanes) is one
    // token, so each row is wholly in or out, and their all-zero chunks would
    // otherwise send the wave through the tiny-tile branch of limb_chunk too.
    auto prep = [&](int slot, char* st) {
      if (!tok) return;
      const int d = limb_shift(row16_max_u32(absmax16(xl[slot], xh[slot])));
      u32x4 o0, o1, o2;
      limb_chunk(xl[slot], xh[slot], d, o0, o1, o2);
      const int r0 = 4 * u;
      *(u32x4*)(st + ((r0 + 0) * 16 + (j ^ (r0 + 0))) * 16) = o0;
      *(u32x4*)(st + ((r0 + 1) * 16 + (j ^ (r0 + 1))) * 16) = o1;
      *(u32x4*)(st + ((r0 + 2) * 16 + (j ^ (r0 + 2))) * 16) = o2;
      if (j == 0) *(int*)(st + kFuseTile + 4 * u) = d - 6;
    };
    // The handoff: the limb writes are done (lgkmcnt(0)), then the barrier
    // without the workgroup fence (which would also wait for the x loads in
    // flight).
    auto handoff = [&]() {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      asm volatile("s_barrier" ::: "memory");
    };
#pragma unroll
    for (int q = 0; q < D; ++q) fetch(q, q);
    prep(0, smem);
    handoff();
    // Iteration i: request k-tile i + D into the slot of tile i, make tile
    // i + 1 into stage (i + 1) & 1 (stage of tile i - 1, released at the
    // previous barrier), hand it over.
    int i = 0;
    for (; i + D <= KT; i += D) {
#pragma unroll
      for (int q = 0; q < D; ++q) {
        fetch(q, i + q + D);
        if (i + q + 1 < KT) prep((q + 1) % D, smem + ((i + q + 1) & 1) * kFuseStage);
        handoff();
      }
    }
#pragma unroll
    for (int q = 0; q < D - 1; ++q) {
      if (i + q < KT) {
        if (i + q + 1 < KT) prep((q + 1) % D, smem + ((i + q + 1) & 1) * kFuseStage);
        handoff();
      }
    }
    return;
  }

  const int r = lane & 15, g = lane >> 4;
  const int strip0 = (blockIdx.x * Ws + wave) * S;
  const int nstrips = min(S, NS - strip0);  // <= 0: the wave only keeps the barriers
  const rsrc_t crs = make_rsrc(codes + (size_t)max(min(strip0, NS - 1), 0) * KT * 64,
                               (uint32_t)max(nstrips, 0) * KT * 1024);
  const rsrc_t srs = make_rsrc(scales + (size_t)max(min(strip0, NS - 1), 0) * KT * 16 * GPT,
                               (uint32_t)max(nstrips, 0) * KT * 16 * GPT * 2);

  auto load = [&](LimbTileStage<S, GPT, 1>& b, int kt) {
    kt = __builtin_amdgcn_readfirstlane(min(kt, KT - 1));
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int se = max(min(s, nstrips - 1), 0);  // absent strips re-read a present one (never stored)
      b.P[s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, lane * 16, (se * KT + kt) * 1024, kAuxNontemporal));
      const int soff = (se * KT + kt) * 16 * GPT * 2;
      if (GPT == 2) {
        b.sw[s][0] = __builtin_amdgcn_raw_buffer_load_b32(srs, r * GPT * 2, soff, 0);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(srs, r * GPT * 2, soff, 0);
        b.sw[s][0] = v[0];
        b.sw[s][1] = v[1];
      }
    }
  };

  float total[S];
#pragma unroll
  for (int s = 0; s < S; ++s) total[s] = 0.f;

  auto compute = [&](const LimbTileStage<S, GPT, 1>& b, const char* st) {
    float part[S];
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      i32x4 af[KBPG];
#pragma unroll
      for (int kk = 0; kk < KBPG; ++kk) {
        const int q = 4 * (gi * KBPG + kk) + g;
        af[kk] = *(const i32x4*)(st + (r * 16 + (q ^ r)) * 16);
      }
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint32_t spair = b.sw[s][gi >> 1];
        const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
        i32x4 acc;
#pragma unroll
        for (int kk = 0; kk < KBPG; ++kk)
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[kk], weights_operand_i8(b.P[s][gi * KBPG + kk]),
                                                      kk == 0 ? i32x4{0, 0, 0, 0} : acc, 0, 0, 0);
        const int low = (int)(((uint32_t)acc[1] << 8) + (uint32_t)acc[0]);  // 256 a1 + a0
        const float v = __builtin_fmaf(65536.0f, (float)acc[2], (float)low);
        part[s] = gi == 0 ? sc * v : __builtin_fmaf(sc, v, part[s]);
      }
    }
    const int dsh = *(const int*)(st + kFuseTile + 4 * g);
#pragma unroll
    for (int s = 0; s < S; ++s) total[s] += __builtin_ldexpf(part[s], dsh);
  };

  LimbTileStage<S, GPT, 1> cb[D];
#pragma unroll
  for (int q = 0; q < D - 1; ++q) load(cb[q], q);
  __syncthreads();
  int i = 0;
  for (; i + D <= KT; i += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int ii = i + q;
      load(cb[(q + D - 1) % D], ii + D - 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(cb[q], smem + (ii & 1) * kFuseStage);
      __syncthreads();
    }
  }
#pragma unroll
  for (int q = 0; q < D - 1; ++q) {
    if (i + q < KT) {  // uniform over the block
      compute(cb[q], smem + ((i + q) & 1) * kFuseStage);
      __syncthreads();
    }
  }

  // Lane (r, g): output row r of each strip for token g.
  if (g < T) {
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < nstrips) y[(size_t)g * N + (strip0 + s) * 16 + r] = total[s];
  }
}

template <int S, int GPT>
hipError_t launch_limbfuse_g(const SmallTArgs& a, const LimbTilePlan& p, hipStream_t st) {
  dim3 grid(p.strip_blocks), block(64 * (p.waves + 1));
  switch (p.depth) {
    case 2:
      hipLaunchKernelGGL((tern_limbfuse_kernel<S, GPT, 2>), grid, block, 0, st, a.x, a.T, a.K,
                         (const u32x4*)a.codes, a.scales, a.y, a.N);
      break;
    case 4:
      hipLaunchKernelGGL((tern_limbfuse_kernel<S, GPT, 4>), grid, block, 0, st, a.x, a.T, a.K,
                         (const u32x4*)a.codes, a.scales, a.y, a.N);
      break;
    default: return hipErrorInvalidValue;
  }
  return (hipError_t)kernel_launched((int)hipGetLastError(), TERN_KERNEL_SMALLT_LIMB_FUSED);
}

template <int RB, int S, int GPT>
hipError_t launch_limbtile_g(const SmallTArgs& a, const LimbTilePlan& p, int8_t* limbs, int* dsh,
                             hipStream_t st) {
  const size_t lds = (size_t)(p.depth + 1) * RB * 16 * 256;
  dim3 grid(p.strip_blocks), block(64 * (p.waves + 1));
  switch (p.depth) {
#define TERN_LIMBTILE_LAUNCH(D)                                                                          \
  case D:                                                                                                \
    hipLaunchKernelGGL((tern_limbtile_kernel<RB, S, GPT, D>), grid, block, lds, st, limbs, dsh, a.T, a.K, \
                       (const u32x4*)a.codes, a.scales, a.y, a.N);                                       \
    break;
    TERN_LIMBTILE_LAUNCH(2)
    case 4:
      // four k-tiles in flight with two strips per wave would spill; the plan
      // takes depth 4 with one strip only
      if constexpr (S == 1) {
        hipLaunchKernelGGL((tern_limbtile_kernel<RB, S, GPT, 4>), grid, block, lds, st, limbs, dsh, a.T, a.K,
                           (const u32x4*)a.codes, a.scales, a.y, a.N);
        break;
      } else {
        return hipErrorInvalidValue;
      }
#undef TERN_LIMBTILE_LAUNCH
    default: return hipErrorInvalidValue;
  }
  return (hipError_t)kernel_launched((int)hipGetLastError(), TERN_KERNEL_SMALLT_LIMB_TILE);
}

template <int RB>
hipError_t launch_limbtile_r(const SmallTArgs& a, const LimbTilePlan& p, int8_t* limbs, int* dsh,
                             hipStream_t st) {
  if (p.strips_per_wave == 1)
    return a.G == 128 ? launch_limbtile_g<RB, 1, 2>(a, p, limbs, dsh, st)
                      : launch_limbtile_g<RB, 1, 4>(a, p, limbs, dsh, st);
  if (p.strips_per_wave == 2)
    return a.G == 128 ? launch_limbtile_g<RB, 2, 2>(a, p, limbs, dsh, st)
                      : launch_limbtile_g<RB, 2, 4>(a, p, limbs, dsh, st);
  return hipErrorInvalidValue;
}

}  // namespace

size_t limbtile_workspace_bytes(int T, int K) {
  const size_t rb = (size_t)(T + 3) / 4;
  const size_t limbs = (rb * 16 * K + 255) & ~(size_t)255;
  return limbs + ((rb * 4 * (K / 256) * 4 + 255) & ~(size_t)255);
}

int launch_limbtile(const SmallTArgs& a, const LimbTilePlan& p, void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (p.waves < 1 || p.waves > 8 || p.strip_blocks < 1) return (int)hipErrorInvalidValue;
  if (p.fused) {
    if (a.T < 1 || a.T > 4) return (int)hipErrorInvalidValue;
    if (p.strips_per_wave == 1)
      return (int)(a.G == 128 ? launch_limbfuse_g<1, 2>(a, p, st) : launch_limbfuse_g<1, 4>(a, p, st));
    if (p.strips_per_wave == 2)
      return (int)(a.G == 128 ? launch_limbfuse_g<2, 2>(a, p, st) : launch_limbfuse_g<2, 4>(a, p, st));
    return (int)hipErrorInvalidValue;
  }
  if (a.T < 1 || a.T > 8 || ws == nullptr) return (int)hipErrorInvalidValue;
  const int RB = (a.T + 3) / 4, slots = 4 * RB;
  int8_t* limbs = (int8_t*)ws;
  int* dsh = (int*)((char*)ws + ((((size_t)RB * 16 * a.K) + 255) & ~(size_t)255));
  const long threads = (long)slots * (a.K / 16);
  hipLaunchKernelGGL(tern_limb_prep_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     a.x, a.T, a.K, slots, limbs, dsh);
  const int e = kernel_launched((int)hipGetLastError(), TERN_KERNEL_SMALLT_LIMB_PREP);
  if (e != 0) return e;
  return (int)(RB == 1 ? launch_limbtile_r<1>(a, p, limbs, dsh, st) : launch_limbtile_r<2>(a, p, limbs, dsh, st));
}

}  // namespace tern
