// tern_kernels.hip -- the per-wave bf16-activation kernel of the
// ternary-weight linear layer on gfx950 (MI355X, CDNA4).
//
// y[t][n] = sum_g s[n][g] * sum_{k in g} w[n][k] * x[t][k], w in {-1,0,+1},
// one fp16 scale per G weights along K ("NInfer sm_89 fork" article, section
// 9 item 2).
//
//  * tern_small_t_kernel -- bf16 activations, one token (TT = 1: the gemv's
//    kernel where its int8 limbs do not fit LDS, or with TERN_TUNE_GEMV=bf16)
//    or a 16-token tile (small_t / small_t_tiled on narrow layers). Streams
//    the 2-bit packed weights with 16-byte loads, turns each code pair into a
//    bf16 pair {0, +-2.0} with one shift and one mask, and lets the
//    v_mfma_f32_16x16x32_bf16 matrix core multiply them with the activation
//    tile. The activation tile is the MFMA A operand (rows = tokens), the
//    weights the B operand (columns = outputs), so each lane's four
//    accumulators share one output row and one scale per group. Each wave
//    owns S 16-row strips over a contiguous K range; the waves of a workgroup
//    split K and are summed in a fixed order through LDS (deterministic).
//
// The other kernels live next to their launchers: the integer-limb gemv and
// resident small-T kernel in tern_limb.hip, the activation-tiled small-T
// kernel in tern_tile.hip, the small-T limb path in tern_limbtile.hip, the
// quantisation and row-major s8 kernels in tern_s8.hip, the operand-order s8
// contraction in tern_s8mma.hip and the bf16 prefill in tern_b16mma.hip.
//
// Packed layout v1 is specified in include/tern.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

// --------------------------------------------------------------------------
// bf16-activation kernel (gemv: TT = 1, small_t / small_t_tiled: TT = 16)
// --------------------------------------------------------------------------
//
// Grid: x = strip blocks (S strips each), y = token tiles (TT = 16) or tokens
// (TT = 1). Block: W waves; wave w streams k-tiles [w*KT/W, (w+1)*KT/W) of
// its S strips. The loads of k-tile kt+1 (codes, scales, activation
// fragments) are issued before the MFMAs of k-tile kt, in two register
// stages, so every wave keeps 2*S KiB of weights in flight.
// Dynamic LDS: W * S * (TT == 16 ? 256 : 16) floats for the reduction.


// One register stage: the codes of S strips for one k-tile, their scales
// and, at TT = 16, the activation fragments of the k-tile's 8 MFMAs.
template <int TT, int S, int GPT>
struct SmallTStage {
  u32x4 P[S];
  uint32_t sw[S][GPT / 2];  // fp16 scale pairs of row (lane & 15)
  bf16x8 xa[TT == 16 ? 8 : 1];
};

// Per-wave constant addressing of the streams.
struct SmallTAddr {
  rsrc_t codes;   // this block's strips (nstrips * KT KiB)
  rsrc_t scales;  // this block's scales
  rsrc_t x;       // this grid row's tokens
  int code_voff;  // lane * 16
  int scale_voff; // (lane & 15) * GPT * 2
  int x_voff;     // TT == 16: lane's A-operand row and k group (past the end for absent rows)
  int KT;
  int nstrips;    // strips of this block that exist (<= S)
};

template <int TT, int S, int GPT>
__device__ __forceinline__ void small_t_load(SmallTStage<TT, S, GPT>& b, const SmallTAddr& a,
                                             int kt, bool valid) {
  // kt is uniform; clamp it into the matrix so that even a dropped load has a
  // sane address, and keep the buffer offsets in scalar registers.
  kt = __builtin_amdgcn_readfirstlane(min(max(kt, 0), a.KT - 1));
  const int cv = valid ? a.code_voff : kOffPastEnd;
  const int sv = valid ? a.scale_voff : kOffPastEnd;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    // The last block may hold fewer than S strips: its missing strips re-read
    // the last existing one (never stored).
    const int se = min(s, a.nstrips - 1);
    b.P[s] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(a.codes, cv, (se * a.KT + kt) * 1024,
                                                     kAuxNontemporal));
    const int soff = (se * a.KT + kt) * 16 * GPT * 2;
    if (GPT == 2) {
      b.sw[s][0] = __builtin_amdgcn_raw_buffer_load_b32(a.scales, sv, soff, 0);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(a.scales, sv, soff, 0);
      b.sw[s][0] = v[0];
      b.sw[s][GPT / 2 - 1] = v[1];
    }
  }
  if (TT == 16) {
    const int xv = valid ? a.x_voff : kOffPastEnd;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      b.xa[m] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(a.x, xv, (kt * 256 + 32 * m) * 2, 0));
  }
}

// One k-tile: S strips x 8 MFMAs and the scale epilogue per group. At TT = 1
// the activation row comes from LDS (xs = the block's staged row).
template <int TT, int S, int GPT>
__device__ __forceinline__ void small_t_compute(const SmallTStage<TT, S, GPT>& b,
                                                f32x4 (&total)[S], const uint16_t* xs, int kt,
                                                int lane) {
  constexpr int MPG = 8 / GPT;  // MFMAs (32 k each) per scale group
  bf16x8 xl[8];
  if (TT == 1) {
    // A-operand row 0 (lanes 0, 16, 32, 48) must hold the token. The other
    // rows only feed output rows that are discarded, so every lane of a
    // 16-lane group reads the same 16 bytes (an LDS broadcast).
    const uint16_t* p = xs + kt * 256 + 8 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < 8; ++m) xl[m] = *(const bf16x8*)(p + 32 * m);
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint4 P = uint4{b.P[s].x, b.P[s].y, b.P[s].z, b.P[s].w};
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mm = 0; mm < MPG; ++mm) {
        const int m = gi * MPG + mm;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(TT == 1 ? xl[m] : b.xa[TT == 1 ? 0 : m],
                                                       weights_operand(P, m), acc, 0, 0, 0);
      }
      const uint32_t spair = b.sw[s][gi >> 1];
      const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
      total[s][0] = __builtin_fmaf(sc, acc[0], total[s][0]);
      if (TT == 16) {  // TT == 1 only uses accumulator 0 of lanes 0..15
        total[s][1] = __builtin_fmaf(sc, acc[1], total[s][1]);
        total[s][2] = __builtin_fmaf(sc, acc[2], total[s][2]);
        total[s][3] = __builtin_fmaf(sc, acc[3], total[s][3]);
      }
    }
  }
}

// Depth of the code prefetch ring: deep where a stage is small (each wave
// needs several KiB in flight to cover the HBM latency), shallow where the
// activation fragments of TT = 16 make a stage large.
template <int TT, int S>
constexpr int small_t_depth() { return TT == 1 ? (S == 1 ? 4 : 3) : (S == 4 ? 2 : 3); }

// Workgroups of up to 16 waves for one strip per wave, up to 8 waves otherwise
// (so the register stages of S = 2 or 4 strips fit without spilling).
template <int S>
constexpr int small_t_max_threads() { return S == 1 ? 1024 : 512; }

template <int TT, int S, int GPT>
__global__ void __launch_bounds__(small_t_max_threads<S>()) tern_small_t_kernel(
    const uint16_t* __restrict__ x, int T, int K, const u32x4* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int N) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int OUT = TT == 16 ? 256 : 16;  // partial sums per strip kept per wave
  constexpr int D = small_t_depth<TT, S>();
  const int lane = threadIdx.x & 63;
  // wave index is uniform across the wave; say so, so that k-tile offsets
  // stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int NS = N >> 4;
  const int KT = K >> 8;
  const int sb = blockIdx.x;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int kt0 = (wave * KT) / W;
  const int kt1 = ((wave + 1) * KT) / W;
  const int nkt = kt1 - kt0;
  const int nstrips = min(S, NS - sb * S);  // strips of this block that exist
  uint16_t* xs = (uint16_t*)smem;                               // TT == 1: K activations
  float* red = (float*)(smem + (TT == 1 ? (size_t)K * 2 : 0));  // reduction area

  SmallTAddr a;
  a.KT = KT;
  a.nstrips = nstrips;
  a.codes = make_rsrc(codes + (size_t)sb * S * KT * 64, (uint32_t)nstrips * KT * 1024);
  a.scales = make_rsrc(scales + (size_t)sb * S * KT * 16 * GPT, (uint32_t)nstrips * KT * 16 * GPT * 2);
  a.code_voff = lane * 16;
  a.scale_voff = r * GPT * 2;
  // Token rows of this grid row. TT == 16: rows t0 .. t0+15 (absent rows read
  // as zeros). TT == 1: one token.
  int tok;
  if (TT == 16) {
    const int t0 = blockIdx.y * 16;
    tok = t0 + r;
    a.x = make_rsrc(x + (size_t)t0 * K, (uint32_t)min(16, T - t0) * K * 2);
    a.x_voff = (r * K + 8 * g) * 2;
  } else {
    tok = blockIdx.y;
    a.x = make_rsrc(x + (size_t)tok * K, (uint32_t)K * 2);
    a.x_voff = 0;
  }

  f32x4 total[S];
#pragma unroll
  for (int s = 0; s < S; ++s) total[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring of D register stages over the wave's k-tiles: the loads of k-tile
  // i + D - 1 are issued before the MFMAs of k-tile i. Loads past the end
  // are dropped (no memory traffic), so every round issues the same loads
  // and the wait before each compute covers exactly the stage it consumes.
  SmallTStage<TT, S, GPT> buf[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j) small_t_load(buf[j], a, kt0 + j, j < nkt);
  if (TT == 1) {
    // The block's token row, staged once into LDS (after the first code
    // loads are in flight).
    for (int c = threadIdx.x; c < (K >> 3); c += blockDim.x)
      *(u32x4*)(xs + 8 * c) =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a.x, c * 16, 0, 0));
    __syncthreads();
  }
  int i = 0;
  for (; i + D <= nkt; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      small_t_load(buf[(j + D - 1) % D], a, kt0 + i + j + D - 1, i + j + D - 1 < nkt);
      // keep the prefetch ahead of the MFMAs: the scheduler must not sink it
      __builtin_amdgcn_sched_barrier(0);
      small_t_compute(buf[j], total, xs, kt0 + i + j, lane);
    }
  }
  const int rem = nkt - i;  // 0 .. D-1 k-tiles left, in buf[0 .. rem-1]
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (j < rem) small_t_compute(buf[j], total, xs, kt0 + i + j, lane);

  // Fixed-order reduction over the waves of the block.
  // Accumulator i of lane l is C[t = 4*(l>>4) + i][n = l & 15].
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (TT == 16) {
      float* dst = red + ((size_t)(wave * S + s) * 64 + lane) * 4;
      dst[0] = total[s][0];
      dst[1] = total[s][1];
      dst[2] = total[s][2];
      dst[3] = total[s][3];
    } else if (lane < 16) {
      red[(wave * S + s) * 16 + lane] = total[s][0];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < S * OUT; e += blockDim.x) {
    const int s = e / OUT;
    const int st = sb * S + s;
    if (st >= NS) continue;
    float sum = 0.f;
    // The codes decode to +-2.0, so every partial is twice the true value;
    // halving the sum is exact.
    if (TT == 16) {
      const int tl = (e % OUT) >> 4;  // token within the tile
      const int nl = e & 15;          // row within the strip
      const int l = nl + 16 * (tl >> 2);
      const int i = tl & 3;
      for (int w = 0; w < W; ++w) sum += red[((size_t)(w * S + s) * 64 + l) * 4 + i];
      const int t = blockIdx.y * 16 + tl;
      if (t < T) y[(size_t)t * N + st * 16 + nl] = 0.5f * sum;
    } else {
      const int nl = e & 15;
      for (int w = 0; w < W; ++w) sum += red[(w * S + s) * 16 + nl];
      y[(size_t)tok * N + st * 16 + nl] = 0.5f * sum;
    }
  }
}

template <int TT, int S>
hipError_t launch_small_t_s(const SmallTArgs& a, const SmallTPlan& p, hipStream_t st) {
  const int NS = a.N / 16;
  dim3 grid((NS + S - 1) / S, p.token_tiles);
  dim3 block(64 * p.waves);
  const size_t lds = (size_t)small_t_lds_bytes(TT, S, p.waves, a.K);
  if (lds > 65536) return hipErrorInvalidConfiguration;
  if (a.G == 128)
    hipLaunchKernelGGL((tern_small_t_kernel<TT, S, 2>), grid, block, lds, st, a.x, a.T, a.K,
                       (const u32x4*)a.codes, a.scales, a.y, a.N);
  else
    hipLaunchKernelGGL((tern_small_t_kernel<TT, S, 4>), grid, block, lds, st, a.x, a.T, a.K,
                       (const u32x4*)a.codes, a.scales, a.y, a.N);
  return (hipError_t)kernel_launched((int)hipGetLastError(),
                                     TT == 1 ? TERN_KERNEL_GEMV_BF16 : TERN_KERNEL_SMALLT_WAVE);
}

template <int TT>
hipError_t launch_small_t_tt(const SmallTArgs& a, const SmallTPlan& p, hipStream_t st) {
  switch (p.strips_per_wave) {
    case 1: return launch_small_t_s<TT, 1>(a, p, st);
    case 2: return launch_small_t_s<TT, 2>(a, p, st);
    case 4: return launch_small_t_s<TT, 4>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int small_t_lds_bytes(int tokens_per_tile, int strips, int waves, int K) {
  return (tokens_per_tile == 1 ? K * 2 : 0) +
         waves * strips * (tokens_per_tile == 16 ? 256 : 16) * (int)sizeof(float);
}

int small_t_max_waves(int tokens_per_tile, int strips, int K) {
  int w = strips == 1 ? 16 : 8;  // launch bounds
  while (w > 0 && small_t_lds_bytes(tokens_per_tile, strips, w, K) > 65536) --w;
  return w;
}

int launch_small_t(const SmallTArgs& a, const SmallTPlan& p, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (p.waves < 1 || p.waves > (p.strips_per_wave == 1 ? 16 : 8) || p.token_tiles < 1)
    return (int)hipErrorInvalidValue;
  if (p.tokens_per_tile == 1) return (int)launch_small_t_tt<1>(a, p, st);
  if (p.tokens_per_tile == 16) return (int)launch_small_t_tt<16>(a, p, st);
  return (int)hipErrorInvalidValue;
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace tern
