// tern_kernels.hip -- gfx950 (MI355X, CDNA4) kernels of the ternary-weight
// linear layer.
//
// y[t][n] = sum_g s[n][g] * sum_{k in g} w[n][k] * x[t][k], w in {-1,0,+1},
// one fp16 scale per G weights along K ("NInfer sm_89 fork" article, section
// 9 item 2). Three kernels:
//
//  * tern_small_t_kernel  -- bf16 activations, T <= 16 per token tile. Streams
//    the 2-bit packed weights with 16-byte loads, turns each code pair into a
//    bf16 pair {0, +-2.0} with one shift and one mask, and lets the
//    v_mfma_f32_16x16x32_bf16 matrix core multiply them with the activation
//    tile. The activation tile is the MFMA A operand (rows = tokens), the
//    weights the B operand (columns = outputs), so each lane's four
//    accumulators share one output row and one scale per group. Each wave
//    owns S 16-row strips over a contiguous K range; the waves of a workgroup
//    split K and are summed in a fixed order through LDS (deterministic).
//  * tern_quant_s8_kernel -- per-token absmax (wavefront DPP reduction), then
//    q = clamp(rne(x / (absmax/127)), +-127) with IEEE division.
//  * tern_s8_kernel       -- int8 activations x ternary weights on
//    v_mfma_i32_16x16x64_i8 into int32 group accumulators, then the fp32
//    scale epilogue total = fma(float(acc), s[n][g], total) per group in
//    ascending order and y = total * scale_t.
//
// Packed layout v1 is specified in include/tern.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tern_internal.h"

namespace tern {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Bf16 pair j (0..7) of a code word: codes at bits 15:14 and 31:30 after the
// shift; 0x4000 = +2.0, 0xC000 = -2.0 (scales are halved to compensate).
__device__ __forceinline__ uint32_t code_pair(uint32_t P, int j) {
  return (P << (2 * j)) & 0xC000C000u;
}

// B operand of MFMA m (0..7) of a 256-wide k-tile from the lane's 4 code words.
__device__ __forceinline__ bf16x8 weights_operand(const uint4& P, int m) {
  const uint32_t word = (m >> 1) == 0 ? P.x : (m >> 1) == 1 ? P.y : (m >> 1) == 2 ? P.z : P.w;
  const int j0 = 4 * (m & 1);
  uint4 b;
  b.x = code_pair(word, j0 + 0);
  b.y = code_pair(word, j0 + 1);
  b.z = code_pair(word, j0 + 2);
  b.w = code_pair(word, j0 + 3);
  return __builtin_bit_cast(bf16x8, b);
}

template <int GPT>
struct ScaleWords;
template <>
struct ScaleWords<2> {  // G = 128: two fp16 per (row, k-tile)
  uint32_t v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *(const uint32_t*)p; }
  __device__ __forceinline__ float get(int gi) const {
    return half_bits_to_float((uint16_t)(gi == 0 ? (v & 0xffffu) : (v >> 16)));
  }
};
template <>
struct ScaleWords<4> {  // G = 64: four fp16 per (row, k-tile)
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *(const uint2*)p; }
  __device__ __forceinline__ float get(int gi) const {
    const uint32_t w = gi < 2 ? v.x : v.y;
    return half_bits_to_float((uint16_t)((gi & 1) ? (w >> 16) : (w & 0xffffu)));
  }
};

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

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [p, p + bytes): loads past the end return zero,
// which is how absent tokens and rows read as zeros without branches.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr int kAuxNontemporal = 2;  // "nt": streamed once, do not keep in cache

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

// A voffset past the end of every resource: the load is dropped and reads 0.
constexpr int kOffPastEnd = 0x40000000;

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

// --------------------------------------------------------------------------
// per-token int8 activation quantisation
// --------------------------------------------------------------------------

// Max over the 64 lanes of a wavefront of non-negative float bit patterns
// (integer order equals float order for them). DPP inside each row of 16
// lanes, then the four row results through readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));  // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));  // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t quant_byte(uint32_t xbits, float sc) {
  const float r = rintf(__uint_as_float(xbits) / sc);  // IEEE division, ties-to-even rounding
  const float c = fminf(fmaxf(r, -127.f), 127.f);
  return (uint32_t)((int)c) & 0xffu;
}

__global__ void __launch_bounds__(256) tern_quant_s8_kernel(const uint16_t* __restrict__ x, int K,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  __shared__ uint32_t wmax[4];
  const int t = blockIdx.x;
  const uint4* xr = (const uint4*)(x + (size_t)t * K);
  const int nchunk = K >> 3;
  uint32_t m = 0;
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = max(m, (w[i] << 16) & 0x7fff0000u);
      m = max(m, w[i] & 0x7fff0000u);
    }
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const uint32_t am = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float a = __uint_as_float(am);
  const float sc = a / 127.0f;  // IEEE single division
  if (threadIdx.x == 0) scale[t] = am == 0 ? 0.0f : sc;
  uint2* qr = (uint2*)(q + (size_t)t * K);
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    uint2 out = uint2{0u, 0u};
    if (am != 0) {
      const uint4 v = xr[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[2 * i] = quant_byte(w[i] << 16, sc);
        b[2 * i + 1] = quant_byte(w[i] & 0xffff0000u, sc);
      }
      out.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      out.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    }
    qr[c] = out;
  }
}

// --------------------------------------------------------------------------
// s8 kernel: int8 activations x ternary weights on the i8 matrix cores
// --------------------------------------------------------------------------
//
// Workgroup tile BM tokens x BN outputs, (BM/WM) x (BN/WN) waves, each wave a
// WM x WN block of 16x16 MFMA tiles. Per 256-wide k-tile the workgroup copies
// the int8 activation tile to LDS and decodes the BN/16 packed weight tiles
// to int8 rows in LDS ([row][k], padded rows of 272 bytes so that 16 rows
// read 16 bytes each without bank conflicts). An i8 MFMA operand slot
// (l >> 4, i) of lane l holds k = 64*kb + 16*(l >> 4) + i for both operands.

constexpr int kS8Pitch = 256 + 16;

// Sign-extend the 2-bit code at bit b of P to an int8 byte.
__device__ __forceinline__ uint32_t code_byte(uint32_t P, int b) {
  return (uint32_t)(((int32_t)(P << (30 - b))) >> 30) & 0xffu;
}

template <int BM, int BN, int WM, int WN, int GPT, bool DEBUG_ACC>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
    tern_s8_kernel(const int8_t* __restrict__ q, const float* __restrict__ act_scale, int T, int K,
                   const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                   float* __restrict__ y, int32_t* __restrict__ acc_out, int N) {
  constexpr int NWN = BN / WN;
  constexpr int NTHR = (BM / WM) * NWN * 64;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int KBPG = 4 / GPT;  // 64-wide k-blocks per scale group
  __shared__ __attribute__((aligned(16))) int8_t As[BM * kS8Pitch];
  __shared__ __attribute__((aligned(16))) int8_t Bs[BN * kS8Pitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int t0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int NS = N >> 4;
  const int KT = K >> 8;
  const int NG = K / (256 / GPT);
  const int r = lane & 15;
  const int g = lane >> 4;

  f32x4 tot[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) tot[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < KT; ++kt) {
    // Activation tile: BM rows x 256 bytes.
    for (int c = tid; c < BM * 16; c += NTHR) {
      const int row = c >> 4, col = (c & 15) * 16;
      uint4 v = uint4{0u, 0u, 0u, 0u};
      if (t0 + row < T) v = *(const uint4*)(q + (size_t)(t0 + row) * K + kt * 256 + col);
      *(uint4*)(As + row * kS8Pitch + col) = v;
    }
    // Weight tiles: BN/16 strips x 256 code words, decoded to int8 rows.
    for (int c = tid; c < (BN / 16) * 256; c += NTHR) {
      const int sl = c >> 8;
      const int win = c & 255;
      const int L = win >> 2, qw = win & 3;
      const int st = (n0 >> 4) + sl;
      const uint32_t P = st < NS ? codes[((size_t)st * KT + kt) * 256 + win] : 0u;
      // word qw holds MFMAs m = 2qw (k = 64qw + 8g' + e) and m = 2qw+1
      // (k = 64qw + 32 + 8g' + e), e = 2d + h at bit (h ? 30 : 14) - 2d (- 8).
      uint32_t lo0 = 0, lo1 = 0, hi0 = 0, hi1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = e >> 1, h = e & 1;
        const int b = (h ? 30 : 14) - 2 * d;
        lo0 |= code_byte(P, b) << (8 * e);
        hi0 |= code_byte(P, b - 8) << (8 * e);
        const int b2 = (h ? 30 : 14) - 2 * (d + 2);
        lo1 |= code_byte(P, b2) << (8 * e);
        hi1 |= code_byte(P, b2 - 8) << (8 * e);
      }
      int8_t* rowp = Bs + (sl * 16 + (L & 15)) * kS8Pitch + 64 * qw + 8 * (L >> 4);
      *(uint2*)(rowp) = uint2{lo0, lo1};
      *(uint2*)(rowp + 32) = uint2{hi0, hi1};
    }
    __syncthreads();

#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      i32x4 acc[TM][TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KBPG; ++kk) {
        const int kb = gi * KBPG + kk;
        i32x4 af[TM], bf[TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
          af[a] = *(const i32x4*)(As + (wm * WM + a * 16 + r) * kS8Pitch + kb * 64 + 16 * g);
#pragma unroll
        for (int b = 0; b < TN; ++b)
          bf[b] = *(const i32x4*)(Bs + (wn * WN + b * 16 + r) * kS8Pitch + kb * 64 + 16 * g);
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
      }
      const int gidx = kt * GPT + gi;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int n = n0 + wn * WN + b * 16 + r;  // accumulator column of this lane
        const int st = n >> 4;
        if (DEBUG_ACC) {
#pragma unroll
          for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = t0 + wm * WM + a * 16 + 4 * g + i;
              if (t < T && st < NS) acc_out[((size_t)t * N + n) * NG + gidx] = acc[a][b][i];
            }
        } else {
          const float sv =
              st < NS ? half_bits_to_float(scales[(((size_t)st * KT + kt) * 16 + r) * GPT + gi])
                      : 0.f;
#pragma unroll
          for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              tot[a][b][i] = __builtin_fmaf((float)acc[a][b][i], sv, tot[a][b][i]);
        }
      }
    }
    __syncthreads();
  }

  if (!DEBUG_ACC) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + wm * WM + a * 16 + 4 * g + i;
        if (t >= T) continue;
        const float as = act_scale[t];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int n = n0 + wn * WN + b * 16 + r;
          if ((n >> 4) < NS) y[(size_t)t * N + n] = tot[a][b][i] * as;
        }
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
  return hipGetLastError();
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

template <int BM, int BN, int WM, int WN>
hipError_t launch_s8_tile(const S8Args& a, hipStream_t st) {
  dim3 grid((a.N + BN - 1) / BN, (a.T + BM - 1) / BM);
  dim3 block((BM / WM) * (BN / WN) * 64);
  const bool dbg = a.acc_out != nullptr;
  if (a.G == 128) {
    if (dbg)
      hipLaunchKernelGGL((tern_s8_kernel<BM, BN, WM, WN, 2, true>), grid, block, 0, st, a.q,
                         a.act_scale, a.T, a.K, (const uint32_t*)a.codes, a.scales, a.y,
                         a.acc_out, a.N);
    else
      hipLaunchKernelGGL((tern_s8_kernel<BM, BN, WM, WN, 2, false>), grid, block, 0, st, a.q,
                         a.act_scale, a.T, a.K, (const uint32_t*)a.codes, a.scales, a.y,
                         a.acc_out, a.N);
  } else {
    if (dbg)
      hipLaunchKernelGGL((tern_s8_kernel<BM, BN, WM, WN, 4, true>), grid, block, 0, st, a.q,
                         a.act_scale, a.T, a.K, (const uint32_t*)a.codes, a.scales, a.y,
                         a.acc_out, a.N);
    else
      hipLaunchKernelGGL((tern_s8_kernel<BM, BN, WM, WN, 4, false>), grid, block, 0, st, a.q,
                         a.act_scale, a.T, a.K, (const uint32_t*)a.codes, a.scales, a.y,
                         a.acc_out, a.N);
  }
  return hipGetLastError();
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

int launch_quant_s8(const uint16_t* x, int T, int K, int8_t* q, float* scale, void* stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(tern_quant_s8_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, x, K, q,
                     scale);
  return (int)hipGetLastError();
}

int launch_s8(const S8Args& a, const S8Plan& p, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (p.bm == 128 && p.bn == 128) return (int)launch_s8_tile<128, 128, 64, 64>(a, st);
  if (p.bm == 64 && p.bn == 64) return (int)launch_s8_tile<64, 64, 32, 32>(a, st);
  if (p.bm == 32 && p.bn == 64) return (int)launch_s8_tile<32, 64, 16, 32>(a, st);
  return (int)hipErrorInvalidValue;
}

const char* hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace tern
