// tern_b16mma.hip -- prefill contraction on bf16 activations (the
// small_t_tiled rung above one 16-token tile, which is where T >= 17 goes
// when the s8 rung is switched off): bf16 activations x ternary weights on
// v_mfma_f32_16x16x32_bf16, fp32 accumulation, fp32 scale epilogue.
//
// y[t][n] = sum_g s[n][g] * sum_{k in g} w[n][k] * x[t][k], w in {-1,0,+1},
// one fp16 scale per G weights along K ("NInfer sm_89 fork" article, section
// 9 item 2). The pages keep a bf16 matrix-core prefill path next to the int8
// one as the control that does not quantise activations ("NINFER ternary
// perf-tuning" notes, sections 2 and 4).
//
// The structure is the s8 contraction's (tern_s8mma.hip) with bf16 operands:
//  * wave tile TB x 16 tokens by S x 16 outputs; a workgroup's 4 waves share
//    one TB x 16-token activation tile in LDS (double-buffered, direct
//    buffer-to-LDS loads) and take S strips each;
//  * the codes decode in registers into bf16 B operands, (word << 2j) &
//    0xC000C000 = two bf16 of value 2w (weights_operand), each decoded
//    operand feeding TB MFMAs; the factor 2 leaves at the store;
//  * per 128-wide group the MFMA chain accumulates the exact products in
//    fp32, and one fma per accumulator folds it into the total with the fp16
//    scale (v_fma_mix_f32), groups in ascending order;
//  * XCD tile order as in the s8 contraction.
// Cost per MFMA (16 cycles on the matrix core): 1 VALU instruction of
// epilogue and 7.5 / TB of decode.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

template <int GPT, int S>
struct B16mStage {
  u32x4 code[S];            // the lane's 16 code bytes of each strip
  uint32_t sw[S][GPT / 2];  // fp16 scale pairs of row (lane & 15)
};

template <int GPT, int TB, int S>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) tern_b16m_kernel(
    const uint16_t* __restrict__ x, int T, int K, const u32x4* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int N, int nx, int ny, int xrows) {
  constexpr int BM = 16 * TB;    // tokens per tile
  constexpr int MPG = 8 / GPT;   // 32-wide k-slices per scale group
  constexpr int LPW = BM / 8;    // 1 KiB activation loads per wave per k-tile
  constexpr int WG_STRIPS = 4 * S;
  // Activation tile: BM rows x 32 chunks of 16 bytes (8 bf16); chunk c of
  // row t sits at position t*32 + (c ^ (t & 15)), so the 16 rows of an
  // operand read fall in different banks.
  __shared__ __attribute__((aligned(1024))) char As[2][BM * 512];

  // Tile (ty, tx): as in the s8 contraction (xrows > 0: XCD-contiguous token
  // tiles, token tile fastest; 0: plain order, output blocks fastest).
  int ty, tx;
  if (xrows) {
    const int xcd = (int)(blockIdx.x & 7), slot = (int)(blockIdx.x >> 3);
    ty = xcd * xrows + slot % xrows;
    tx = slot / xrows;
  } else {
    ty = (int)blockIdx.x / nx;
    tx = (int)blockIdx.x - ty * nx;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int NS = N >> 4, KT = K >> 8;
  const int t0 = ty * BM;
  const int nt = min(BM, T - t0);
  const int st0 = tx * WG_STRIPS + wave * S;  // first strip of this wave
  const int nst = max(0, min(S, NS - st0));   // of which exist

  const rsrc_t xr = make_rsrc(x + (size_t)t0 * K, (uint32_t)nt * K * 2);
  const rsrc_t cr = make_rsrc(codes + (size_t)min(st0, NS) * KT * 64, (uint32_t)nst * KT * 1024);
  const rsrc_t sr = make_rsrc(scales + (size_t)min(st0, NS) * KT * 16 * GPT,
                              (uint32_t)nst * KT * 16 * GPT * 2);

  // Activation tile kt into buffer buf: load j of wave w covers positions
  // [64(w*LPW + j), +64), i.e. rows 2(w*LPW + j) and the next; lane l writes
  // position 64(w*LPW + j) + l and fetches that row's global chunk
  // (l & 31) ^ (row & 15). Rows past the last token read as zeros.
  auto stage_a = [&](int kt, int buf) {
    kt = __builtin_amdgcn_readfirstlane(kt);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int ld = wave * LPW + j;
      const int row = 2 * ld + (lane >> 5);
      const int chunk = (lane & 31) ^ (row & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (__attribute__((address_space(3))) void*)&As[buf][ld * 1024], 16, row * K * 2 + chunk * 16,
          kt * 512, 0, 0);
    }
  };
  auto load_w = [&](int kt, B16mStage<GPT, S>& b) {
    kt = __builtin_amdgcn_readfirstlane(kt);
#pragma unroll
    for (int c = 0; c < S; ++c) {
      const int ce = min(c, max(nst - 1, 0));
      b.code[c] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, lane * 16, (ce * KT + kt) * 1024, kAuxNontemporal));
      const int soff = (ce * KT + kt) * 16 * GPT * 2;
      if (GPT == 2) {
        b.sw[c][0] = __builtin_amdgcn_raw_buffer_load_b32(sr, r * GPT * 2, soff, 0);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(sr, r * GPT * 2, soff, 0);
        b.sw[c][0] = v[0];
        b.sw[c][1] = v[1];
      }
    }
  };

  f32x4 tot[TB][S];
#pragma unroll
  for (int a = 0; a < TB; ++a)
#pragma unroll
    for (int c = 0; c < S; ++c) tot[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One k-tile: per scale group, the A fragments of its k-slices (shared by
  // the S strips), then per strip MPG x TB MFMAs and the group's epilogue.
  auto compute = [&](int buf, const B16mStage<GPT, S>& b) {
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      bf16x8 af[MPG][TB];
#pragma unroll
      for (int mm = 0; mm < MPG; ++mm)
#pragma unroll
        for (int a = 0; a < TB; ++a) {
          const int m = gi * MPG + mm;
          const int row = a * 16 + r;  // row & 15 == r
          af[mm][a] = *(const bf16x8*)&As[buf][row * 512 + (((4 * m + g) ^ r) << 4)];
        }
#pragma unroll
      for (int c = 0; c < S; ++c) {
        const uint4 P = uint4{b.code[c][0], b.code[c][1], b.code[c][2], b.code[c][3]};
        f32x4 acc[TB];
#pragma unroll
        for (int mm = 0; mm < MPG; ++mm) {
          const bf16x8 bf = weights_operand(P, gi * MPG + mm);
#pragma unroll
          for (int a = 0; a < TB; ++a)
            acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mm][a], bf,
                                                             mm == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[a], 0, 0, 0);
        }
        const uint32_t sp = b.sw[c][gi >> 1];
        const float sv = half_bits_to_float((uint16_t)((gi & 1) ? (sp >> 16) : (sp & 0xffffu)));
#pragma unroll
        for (int a = 0; a < TB; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) tot[a][c][e] = __builtin_fmaf(sv, acc[a][e], tot[a][c][e]);
      }
    }
  };

  // Pipeline as in the s8 contraction: one barrier per k-tile, k-tiles in
  // pairs (buffers 0 then 1) without an exit in between; the loads of k-tile
  // kt+1 go out before the MFMAs of k-tile kt.
  B16mStage<GPT, S> wA, wB;
  stage_a(0, 0);
  load_w(0, wA);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= KT; kt += 2) {
    stage_a(kt + 1, 1);
    load_w(kt + 1, wB);
    __builtin_amdgcn_sched_barrier(0);
    compute(0, wA);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int k2 = min(kt + 2, KT - 1);
    stage_a(k2, 0);
    load_w(k2, wA);
    __builtin_amdgcn_sched_barrier(0);
    compute(1, wB);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (kt < KT) compute(0, wA);

  // Accumulator e of lane l: token t0 + 16a + 4(l >> 4) + e, output row
  // (l & 15) of each strip; 0.5 undoes the +-2 decode.
#pragma unroll
  for (int a = 0; a < TB; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tl = a * 16 + 4 * g + e;
      if (tl >= nt) continue;
#pragma unroll
      for (int c = 0; c < S; ++c)
        if (c < nst) y[(size_t)(t0 + tl) * N + (st0 + c) * 16 + r] = 0.5f * tot[a][c][e];
    }
}

template <int GPT, int TB, int S>
hipError_t launch_b16m_t(const SmallTArgs& a, bool xcd_order, hipStream_t st) {
  constexpr int WG_STRIPS = 4 * S;
  const int NS = a.N / 16;
  const int nx = (NS + WG_STRIPS - 1) / WG_STRIPS;
  const int ny = (a.T + 16 * TB - 1) / (16 * TB);
  const int xrows = (xcd_order && ny % 8 == 0) ? ny / 8 : 0;
  hipLaunchKernelGGL((tern_b16m_kernel<GPT, TB, S>), dim3(nx * ny), dim3(256), 0, st, a.x, a.T, a.K,
                     (const u32x4*)a.codes, a.scales, a.y, a.N, nx, ny, xrows);
  return (hipError_t)kernel_launched((int)hipGetLastError(), TERN_KERNEL_B16_PREFILL);
}

template <int GPT>
hipError_t launch_b16m_g(const SmallTArgs& a, int tb, int s, bool x, hipStream_t st) {
  switch (tb * 16 + s) {
    case 2 * 16 + 1: return launch_b16m_t<GPT, 2, 1>(a, x, st);
    case 4 * 16 + 1: return launch_b16m_t<GPT, 4, 1>(a, x, st);
    case 2 * 16 + 2: return launch_b16m_t<GPT, 2, 2>(a, x, st);
    case 2 * 16 + 4: return launch_b16m_t<GPT, 2, 4>(a, x, st);
    case 4 * 16 + 2: return launch_b16m_t<GPT, 4, 2>(a, x, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int launch_b16_prefill(const SmallTArgs& a, const S8Plan& p, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.T < 1) return (int)hipErrorInvalidValue;
  // 8 blocks would not fit the registers; 3 (the s8 plan's 48-token tile) runs as 4.
  // The s8 plan's 64 x 64 wave tile runs as 64 x 32 here: its bf16 A fragments
  // take twice the s8 ones' registers, and at 64 x 64 the kernel spilled (the
  // two ran gate_up at T = 2048 in the same time on MI355X, 702 against 704 us).
  const int tb = p.token_blocks > 2 ? 4 : p.token_blocks;
  const int s = tb == 4 && p.strips > 2 ? 2 : p.strips;
  return (int)(a.G == 128 ? launch_b16m_g<2>(a, tb, s, p.xcd_order, st)
                          : launch_b16m_g<4>(a, tb, s, p.xcd_order, st));
}

}  // namespace tern
