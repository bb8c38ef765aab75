// tern_limb.hip -- decode kernel on the gfx950 integer matrix cores: the
// T = 1 gemv rung, and the small_t rung for short batches (tokens in their
// own lane groups, TT = 4 and 8 below).
//
// y[t][n] = sum_g s[n][g] * sum_{k in g} w[n][k] * x[t][k], w in {-1,0,+1},
// one fp16 scale per G weights along K ("NInfer sm_89 fork" article, section
// 9 item 2); T = 1 is the decode rung of the rung map ("NINFER ternary
// perf-tuning" notes, section 2).
//
// At T = 1 the layer reads every weight once and does one multiply-add with
// it, so what competes with the HBM stream is turning packed codes into
// matrix-core operands (the notes, section 6, measure that decode arithmetic
// as a quarter of the kernel time on their card). Decoded as int8 for
// v_mfma_i32_16x16x64_i8, a 32-bit code word becomes four operand registers
// with one AND and three shift+AND pairs -- 7 ALU operations per 16 weights,
// against 15 for bf16 operands.
//
// The bf16 activations then have to enter the integer MFMA exactly. Every
// 256-wide k-tile of a token is turned into fixed point relative to its own
// largest magnitude: with 2^E <= max|x| < 2^(E+1) over the tile and d = E - 21,
// v = rne(x * 2^-d) is an integer with |v| <= 2^22, exact for every activation
// within 2^14 of the tile maximum (bf16 carries 8 significant bits) and within
// 2^(d-1) <= 2^-22 * max|x| otherwise. v is split into three balanced int8
// limbs v = l0 + 256 l1 + 65536 l2 (l0, l1 in [-128, 127], |l2| <= 64) that
// occupy A rows 3t, 3t+1, 3t+2, so five tokens fit one 16-row operand. The
// MFMA sums 64 * w * l exactly in int32 (codes decode to +-64), and per scale
// group the fp32 epilogue adds s * 2^(d - 6 + 8L) * acc to the total of row
// 3t + L, so that every partial sum carries its true magnitude (this keeps
// tiny activations out of the fp32 denormal range). At the end
//   y[t][n] = (R[3t+2] + R[3t+1]) + R[3t]
// with R the per-row fp32 totals. The only approximations are the fixed-point
// rounding above and fp32 accumulation over the groups; the integer part is
// exact (the mixed-format fp8/fp4 matrix core would decode cheaper still, but
// it sums each run of 8 products with about 13 bits below their largest one,
// which loses small activations next to large ones).
//
// Operand order: limb rows are stored in LDS in the order of the s8 rung's
// quantised activations (include/tern.h, TERN_Q_OPERAND_ORDER): inside each
// 64-wide k-block, byte 16g + 4i + e holds k = 8g + m(i, e), m(i, .) =
// {32+2i, 2i, 33+2i, 2i+1}, which is how weights_operand_i8 lays out the codes
// of packed layout v1. Lane 16g + r then reads its 16-byte A operand for
// k-block b at row r, offset 64b + 16g.
//
// Base-3 weights (layout t5, include/tern.h; L5 = true, T = 1 only). Five
// weights per byte ("NInfer sm_89 fork" article, section 9 item 2): a lane's
// 64 weights of a k-tile are three words of five-trit bytes (60 weights) and
// a tail byte of four 2-bit trits. A word splits into its even and odd bytes
// in 16-bit lanes; five times "multiply by 3" moves the next trit (t = w + 1)
// of every byte into bits 8-9 of its lane, and one byte permute gathers the
// four trits into an int8 operand register (about 5 VALU instructions per 4
// weights, against 7 per 16 for the 2-bit layout). The MFMA then sums
// t * limb = w * limb + limb; each scale group's accumulators start from
// minus the group's limb sums (made once per workgroup in the prep, kept in
// LDS), so the accumulators are exactly those of the 2-bit path without its
// 64x factor.
//
// Work split. A workgroup owns Wn*S strips of 16 outputs over the whole K; its
// Wn*Wk waves take S strips each over a 1/Wk share of the k-tiles (wide layers
// use Wk = 1, narrow ones split K so that enough waves stream). Each wave keeps
// D k-tiles of codes in flight; the partial sums of the Wk shares are added
// through LDS in a fixed order (deterministic, no atomics).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

template <int S>
struct LimbStage {
  u32x4 P[S];  // the lane's 16 code bytes of each of the wave's strips
};

// TT: 1 (single token: rows 0..2), 5 (T <= 5 tokens: A row r = limb row r)
// or 4 / 8 (T <= 4 / 8 tokens, one / two A operands: row 4u + L of operand b
// reads token 4b + u's limb L, so lane group u holds tokens u and 4 + u and
// combines each one's three limbs as at TT = 1; rows 4u + 3 and those of
// absent tokens read some stored row and only feed accumulators that are not
// stored).
// Dynamic LDS (limb_lds_bytes): 3T limb rows of K + 64 bytes, the tile
// exponents d [T][K/256] (int), then the workgroup's scales in their packed
// order [strip][k-tile][row][group]; all of it is reused for the final
// reduction.
// Trits t = w + 1 of a t5 k-tile as four int8 operand quads (registers
// R = 4q + i for MFMA q): R = 5w + d from word w, digit d; R = 15 from the
// tail byte j of P.w.
__device__ __forceinline__ void t5_operands(const u32x4& P, int j, i32x4 (&op)[4]) {
  uint32_t reg[16];
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    uint32_t E = __builtin_amdgcn_perm(P[w], P[w], 0x0c020c00u);  // bytes 0, 2 in 16-bit lanes
    uint32_t O = __builtin_amdgcn_perm(P[w], P[w], 0x0c030c01u);  // bytes 1, 3
#pragma unroll
    for (int d = 0; d < 5; ++d) {
      const uint32_t E3 = E * 3u, O3 = O * 3u;  // no carry out of a lane: 3 * 255 < 2^16
      reg[5 * w + d] = __builtin_amdgcn_perm(O3, E3, 0x07030501u);  // [E3.1, O3.1, E3.3, O3.3]
      if (d < 4) {
        E = E3 & 0x00ff00ffu;
        O = O3 & 0x00ff00ffu;
      }
    }
  }
  const uint32_t tb = (P[3] >> (8 * j)) & 0xffu;
  uint32_t x = (tb << 6) | tb;
  x = (x << 12) | x;  // bits 2e..2e+1 of tb at bits 8e..8e+1
  reg[15] = x & 0x03030303u;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    op[q] = i32x4{(int)reg[4 * q], (int)reg[4 * q + 1], (int)reg[4 * q + 2], (int)reg[4 * q + 3]};
}

template <int TT, int S, int GPT, int D, bool L5>
__global__ void __launch_bounds__(1024) tern_limb_kernel(
    const uint16_t* __restrict__ x, int T, int K, const u32x4* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int N, int Wn, int Wk) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  static_assert(GPT == 2 || GPT == 4, "G must be 128 or 64");
  static_assert(!L5 || (TT == 1 && S == 1), "layout t5: one token, one strip per wave");
  constexpr int KBPG = 4 / GPT;  // 64-wide k-blocks per scale group
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nth = blockDim.x;
  const int NS = N >> 4, KT = K >> 8;
  const int wn = wave % Wn, wk = wave / Wn;
  const int strip0 = (blockIdx.x * Wn + wn) * S;
  const int nstrips = min(S, NS - strip0);  // <= 0: this wave only helps with the activations
  const int kt0 = (wk * KT) / Wk;
  const int nkt = ((wk + 1) * KT) / Wk - kt0;
  const int NR = 3 * T;  // A rows in use
  const int rs = K + 64;  // LDS bytes per limb row; the 64-byte pad puts the 12
                          // A-operand reads of rows 0..2 on distinct banks
  const int r = lane & 15, g = lane >> 4;
  const int SB = Wn * S;                      // strips of the workgroup
  const int wstrip0 = blockIdx.x * SB;
  const int nsb = min(SB, NS - wstrip0);      // of which exist
  int* dexp = (int*)(smem + (size_t)NR * rs);  // [T][KT]
  char* lsc = smem + (size_t)NR * rs + (size_t)T * KT * 4;  // [SB][KT][16][GPT] fp16
  // t5: per scale group {-S0, -S1, -S2, 0}, S_L the sum of limb L over the group
  int* gbias = (int*)(lsc + (size_t)SB * KT * 16 * GPT * 2);  // [KT * GPT][4]

  const rsrc_t xr = make_rsrc(x, (uint32_t)T * K * 2);
  // The workgroup's scales, 16-byte chunks (2*GPT per strip and k-tile).
  const int nsc = nsb * KT * 2 * GPT;
  const rsrc_t wsr = make_rsrc(scales + (size_t)wstrip0 * KT * 16 * GPT, (uint32_t)nsc * 16);

  // 1. The activations are requested first, so that they do not queue behind
  //    the weight stream. Chunk c covers token c / (K/16), k-block j >> 2 and
  //    lane group j & 3 (j = c mod K/16): natural k = 64(j>>2) + 8(j&3) + 0..7
  //    (lo) and + 32 (hi). The 16 chunks of a k-tile sit in one DPP row.
  const int KC16 = K >> 4;
  const int nchunk = T * KC16;
  auto chunk_x = [&](int c, u32x4& lo, u32x4& hi) {
    const int t = c / KC16, j = c - t * KC16;
    const int base = t * K + 64 * (j >> 2) + 8 * (j & 3);
    lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, base * 2, 0, 0));
    hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (base + 32) * 2, 0, 0));
  };
  // Up to two chunks and two scale chunks per thread are requested up front.
  u32x4 xpre[2][2], spre[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (tid + it * nth < nchunk) chunk_x(tid + it * nth, xpre[it][0], xpre[it][1]);
    if (tid + it * nth < nsc)
      spre[it] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wsr, (tid + it * nth) * 16, 0, 0));
  }

  // 2. Weight prefetch ring: the first D - 1 k-tiles of this wave's strips.
  //    (The codes are read once: non-temporal.)
  const int sclamp = max(min(strip0, NS - 1), 0);
  constexpr int kStripTileBytes = L5 ? 832 : 1024;  // code bytes per strip and k-tile
  const rsrc_t crs = make_rsrc((const char*)codes + (size_t)sclamp * KT * kStripTileBytes,
                               (uint32_t)max(nstrips, 0) * KT * kStripTileBytes);
  auto load = [&](LimbStage<S>& b, int i) {
    const int kt = __builtin_amdgcn_readfirstlane(min(kt0 + i, KT - 1));
    if constexpr (L5) {
      // block of 4 k-tiles: 4 x 768 bytes of main words, then 256 bytes of tails
      const int blk = (kt >> 2) * 3328;
      const int cm = i < nkt ? lane * 12 : kOffPastEnd;
      const int ct = i < nkt ? 3072 + lane * 4 : kOffPastEnd;
      const auto m = __builtin_amdgcn_raw_buffer_load_b96(crs, cm, blk + 768 * (kt & 3), kAuxNontemporal);
      const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(crs, ct, blk, 0);  // shared by 4 k-tiles
      b.P[0] = u32x4{m[0], m[1], m[2], t};
    } else {
      const int cv = i < nkt ? lane * 16 : kOffPastEnd;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int se = max(min(s, nstrips - 1), 0);
        b.P[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               crs, cv, (se * KT + kt) * 1024, kAuxNontemporal));
      }
    }
  };
  LimbStage<S> ring[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j) load(ring[j], j);

  // 3. Limbs into LDS: per chunk, the k-tile maximum over its DPP row, the
  //    exponent shift d, then three 16-byte limb chunks (rows 3t + L, byte
  //    offset 16j). Rows of 16 lanes are wholly inside or outside [0, nchunk)
  //    since nchunk and the thread count are multiples of 16.
  for (int c0 = 0; c0 < nchunk; c0 += nth) {
    const int c = c0 + tid;
    u32x4 lo, hi;
    if (c0 == 0) {
      lo = xpre[0][0];
      hi = xpre[0][1];
    } else if (c0 == nth) {
      lo = xpre[1][0];
      hi = xpre[1][1];
    } else if (c < nchunk) {
      chunk_x(c, lo, hi);
    }
    if (c < nchunk) {
      const int d = limb_shift(row16_max_u32(absmax16(lo, hi)));
      const int t = c / KC16, j = c - t * KC16;
      u32x4 out0, out1, out2;
      limb_chunk(lo, hi, d, out0, out1, out2);
      if constexpr (L5) {
        // limb sums of the chunk, then of its scale group (8 or 4 chunks,
        // consecutive lanes of the DPP row): S_L = sum of limb L over the group
        int sl[3] = {0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sl[0] = __builtin_amdgcn_sdot4((int)out0[e], 0x01010101, sl[0], false);
          sl[1] = __builtin_amdgcn_sdot4((int)out1[e], 0x01010101, sl[1], false);
          sl[2] = __builtin_amdgcn_sdot4((int)out2[e], 0x01010101, sl[2], false);
        }
#pragma unroll
        for (int L = 0; L < 3; ++L) {
          sl[L] += __builtin_amdgcn_update_dpp(0, sl[L], 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
          sl[L] += __builtin_amdgcn_update_dpp(0, sl[L], 0x4e, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
          if (GPT == 2) sl[L] += __builtin_amdgcn_update_dpp(0, sl[L], 0x141, 0xf, 0xf, false);  // row_half_mirror
        }
        constexpr int kChunksPerGroup = 16 / GPT;
        if ((j & (kChunksPerGroup - 1)) == 0)
          *(i32x4*)(gbias + 4 * (j / kChunksPerGroup)) = i32x4{-sl[0], -sl[1], -sl[2], 0};
      }
      char* row = smem + (size_t)(3 * t) * rs + 16 * j;
      *(u32x4*)row = out0;
      *(u32x4*)(row + rs) = out1;
      *(u32x4*)(row + 2 * rs) = out2;
      if ((j & 15) == 0) dexp[t * KT + (j >> 4)] = d;
    }
  }
  for (int c = tid; c < nsc; c += nth) {
    const u32x4 v = c < nth ? spre[0]
                  : c < 2 * nth ? spre[1]
                                : __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wsr, c * 16, 0, 0));
    *(u32x4*)(lsc + 16 * c) = v;
  }
  __syncthreads();

  // 4. Main loop. Lanes whose A row is unused (r >= NR) read row 0 again;
  //    their output rows are never read. Row q of this lane's accumulators
  //    (q = 4g + e) belongs to token q / 3.
  f32x4 total[S];
#pragma unroll
  for (int s = 0; s < S; ++s) total[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr bool TL = TT == 4 || TT == 8;  // token per lane group
  constexpr int RB = TT == 8 ? 2 : 1;       // A operands (row blocks)
  auto token_row = [&](int u) { return u < T ? 3 * u + min(r & 3, 2) : 0; };
  const int arow = TL ? token_row(r >> 2) : (r < NR ? r : 0);
  const char* abase = smem + (size_t)arow * rs + 16 * g;
  const char* abase1 = smem + (size_t)(RB == 2 ? token_row(4 + (r >> 2)) : 0) * rs + 16 * g;
  int tok[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) tok[e] = TT == 1 ? 0 : min((4 * g + e) / 3, T - 1);
  // Scales of this wave's strips in LDS: strip s, k-tile kt, row r.
  const char* wsc = lsc + ((size_t)(wn * S) * KT * 16 + r) * GPT * 2;
  auto compute = [&](const LimbStage<S>& b, int i) {
    const int kt = kt0 + i;
    i32x4 a[4], a1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = *(const i32x4*)(abase + 64 * (4 * kt + q));
    if (RB == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) a1[q] = *(const i32x4*)(abase1 + 64 * (4 * kt + q));
    }
    // TT = 1: the three limbs of the token are accumulators 0..2 of lanes
    // 0..15. Per group they are combined as 65536 a2 + (256 a1 + a0), the
    // bracket exact in int32 (|a_L| <= 2^20), and scaled; the groups of the
    // k-tile are summed first and 2^(d - 6), which undoes the fixed point and
    // the 64x code decode, is applied once per k-tile.
    // TT = 5: each row keeps its own total, scaled by 2^(d - 6 + 8L) (limb
    // L = row mod 3) so that every partial sum carries its true magnitude.
    int dsh[4];
    if (TT == 1) {
      dsh[0] = dexp[kt] - (L5 ? 0 : 6);  // the 2-bit operands carry 64 w
    } else if (TL) {
      dsh[0] = dexp[min(g, T - 1) * KT + kt] - 6;
      if (RB == 2) dsh[1] = dexp[min(g + 4, T - 1) * KT + kt] - 6;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dsh[e] = dexp[tok[e] * KT + kt] - 6 + 8 * ((4 * g + e) % 3);
    }
    i32x4 op5[4];
    if constexpr (L5) t5_operands(b.P[0], kt & 3, op5);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const u32x4 P = b.P[s];
      uint32_t sw[GPT / 2];
      const char* sp = wsc + ((size_t)s * KT + kt) * 16 * GPT * 2;
      if (GPT == 2) {
        sw[0] = *(const uint32_t*)sp;
      } else {
        const uint2 v = *(const uint2*)sp;
        sw[0] = v.x;
        sw[GPT / 2 - 1] = v.y;
      }
      float part = 0.f, part1 = 0.f;  // TT = 1, 4, 8: this k-tile's groups, before 2^(d - 6)
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        i32x4 acc = i32x4{0, 0, 0, 0}, acc1 = acc;
        if constexpr (L5) acc = *(const i32x4*)(gbias + 4 * (kt * GPT + gi));  // minus the limb sums
#pragma unroll
        for (int kk = 0; kk < KBPG; ++kk) {
          const int q = gi * KBPG + kk;
          const i32x4 bq = L5 ? op5[q] : weights_operand_i8(P[q]);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[q], bq, acc, 0, 0, 0);
          if (RB == 2) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[q], bq, acc1, 0, 0, 0);
        }
        const uint32_t spair = sw[gi >> 1];
        const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
        if (TT != 5) {
          const int low = (int)(((uint32_t)acc[1] << 8) + (uint32_t)acc[0]);  // 256 a1 + a0
          const float v = __builtin_fmaf(65536.0f, (float)acc[2], (float)low);
          part = gi == 0 ? sc * v : __builtin_fmaf(sc, v, part);
          if (RB == 2) {
            const int low1 = (int)(((uint32_t)acc1[1] << 8) + (uint32_t)acc1[0]);
            const float v1 = __builtin_fmaf(65536.0f, (float)acc1[2], (float)low1);
            part1 = gi == 0 ? sc * v1 : __builtin_fmaf(sc, v1, part1);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            total[s][e] = __builtin_fmaf(sc, __builtin_ldexpf((float)acc[e], dsh[e]), total[s][e]);
        }
      }
      if (TT != 5) total[s][0] += __builtin_ldexpf(part, dsh[0]);
      if (RB == 2) total[s][1] += __builtin_ldexpf(part1, dsh[1]);
    }
  };
  int i = 0;
  for (; i + D <= nkt; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      load(ring[(j + D - 1) % D], i + j + D - 1);
      // keep the prefetch ahead of the MFMAs: the scheduler must not sink it
      __builtin_amdgcn_sched_barrier(0);
      compute(ring[j], i + j);
    }
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (i + j < nkt) compute(ring[j], i + j);

  // 5. y. Accumulator e of lane l is row 4(l >> 4) + e, column l & 15. With
  //    one token and no K split, lanes 0..15 hold finished outputs. Otherwise
  //    a fixed-order reduction over the Wk shares through LDS (the limbs,
  //    exponents and scales are no longer read).
  if (TT == 1 && Wk == 1) {
    if (lane < 16) {
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (s < nstrips) y[(size_t)(strip0 + s) * 16 + lane] = total[s][0];
    }
    return;
  }
  if (TL) {  // lane group g holds the outputs of tokens g and (RB = 2) 4 + g
    if (Wk == 1) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
        if (4 * b + g < T) {
#pragma unroll
          for (int s = 0; s < S; ++s)
            if (s < nstrips) y[(size_t)(4 * b + g) * N + (strip0 + s) * 16 + r] = total[s][b];
        }
      return;
    }
    // The Wk shares through LDS ([Wk][Wn*S strips][4 RB tokens][16 columns]),
    // added in ascending order.
    __syncthreads();
    float* red4 = (float*)smem;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int b = 0; b < RB; ++b)
        if (4 * b + g < T) red4[(((size_t)wk * SB + wn * S + s) * 4 * RB + 4 * b + g) * 16 + r] = total[s][b];
    __syncthreads();
    const int nout4 = T * SB * 16;
    for (int e = tid; e < nout4; e += nth) {
      const int t = e / (SB * 16);
      const int rem = e - t * (SB * 16);
      const int ls = rem >> 4, col = rem & 15;
      const int st = blockIdx.x * SB + ls;
      if (st >= NS) continue;
      float sum = 0.f;
      for (int w = 0; w < Wk; ++w) sum += red4[(((size_t)w * SB + ls) * 4 * RB + t) * 16 + col];
      y[(size_t)t * N + st * 16 + col] = sum;
    }
    return;
  }
  __syncthreads();
  float* red = (float*)smem;  // [Wk][Wn*S strips][16 rows][16 columns]
#pragma unroll
  for (int s = 0; s < S; ++s) {
    float* dst = red + (((size_t)wk * SB + wn * S + s) * 16 + 4 * g) * 16 + r;
    if (TT == 1) {
      // the whole token sits in row 0 already (rows 1, 2 are zero)
      if (g == 0) {
        dst[0] = total[s][0];
        dst[16] = 0.f;
        dst[32] = 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * g + e < NR) dst[e * 16] = total[s][e];
    }
  }
  __syncthreads();
  const int nout = T * SB * 16;
  for (int e = tid; e < nout; e += nth) {
    const int t = e / (SB * 16);
    const int rem = e - t * (SB * 16);
    const int ls = rem >> 4, col = rem & 15;
    const int st = blockIdx.x * SB + ls;
    if (st >= NS) continue;
    float sum = 0.f;
    for (int w = 0; w < Wk; ++w) {
      const float* src = red + (((size_t)w * SB + ls) * 16 + 3 * t) * 16 + col;
      sum += (src[32] + src[16]) + src[0];
    }
    y[(size_t)t * N + st * 16 + col] = sum;
  }
}

template <int TT, int S, int GPT, bool L5 = false>
hipError_t launch_limb_g(const SmallTArgs& a, const LimbPlan& p, hipStream_t st) {
  const int NS = a.N / 16;
  dim3 grid((NS + p.wn * S - 1) / (p.wn * S));
  dim3 block(64 * p.wn * p.wk);
  const size_t lds = (size_t)limb_lds_bytes(a.T, a.K, a.G, p);
  switch (p.depth) {
#define TERN_LIMB_LAUNCH(D)                                                                        \
  case D:                                                                                          \
    hipLaunchKernelGGL((tern_limb_kernel<TT, S, GPT, D, L5>), grid, block, lds, st, a.x, a.T, a.K, \
                       (const u32x4*)a.codes, a.scales, a.y, a.N, p.wn, p.wk);                     \
    break;
    TERN_LIMB_LAUNCH(2)
    TERN_LIMB_LAUNCH(4)
    TERN_LIMB_LAUNCH(8)
#undef TERN_LIMB_LAUNCH
    default: return hipErrorInvalidValue;
  }
  // the gemv rung (any T <= 5, limbs made per k-tile) or the resident small-T plan
  return (hipError_t)kernel_launched((int)hipGetLastError(),
                                     L5 ? TERN_KERNEL_GEMV_T5
                                        : p.resident ? TERN_KERNEL_SMALLT_RESIDENT : TERN_KERNEL_GEMV_LIMB);
}

template <int TT, int S>
hipError_t launch_limb_s(const SmallTArgs& a, const LimbPlan& p, hipStream_t st) {
  return a.G == 128 ? launch_limb_g<TT, S, 2>(a, p, st) : launch_limb_g<TT, S, 4>(a, p, st);
}

// One strip per wave only: with two or four strips the k-tiles of codes in
// flight no longer fit the registers at 1024 threads per workgroup and the
// kernel spills (measured no faster before the spills either).
template <int TT>
hipError_t launch_limb_t(const SmallTArgs& a, const LimbPlan& p, hipStream_t st) {
  if (p.strips_per_wave != 1) return hipErrorInvalidValue;
  return launch_limb_s<TT, 1>(a, p, st);
}

}  // namespace

int limb_lds_bytes(int T, int K, int G, const LimbPlan& p) {
  const size_t SB = (size_t)p.wn * p.strips_per_wave;
  const size_t main = (size_t)3 * T * (K + 64) + (size_t)T * (K / 256) * 4 + SB * (K / 256) * 16 * (256 / G) * 2 +
                      (p.t5 ? (size_t)(K / G) * 16 : 0);
  const size_t red = (size_t)p.wk * SB * 256 * 4;
  return (int)std::max(main, red);
}

int launch_limb(const SmallTArgs& a, const LimbPlan& p, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int W = p.wn * p.wk;
  if (p.t5) {  // base-3 weights: the single-token gemv, one strip per wave
    if (a.T != 1 || p.strips_per_wave != 1 || p.token_lanes || p.resident || a.K % 1024 != 0 || p.wn < 1 ||
        p.wk < 1 || W > 16 || limb_lds_bytes(1, a.K, a.G, p) > kLimbMaxLds)
      return (int)hipErrorInvalidValue;
    return (int)(a.G == 128 ? launch_limb_g<1, 1, 2, true>(a, p, st) : launch_limb_g<1, 1, 4, true>(a, p, st));
  }
  if (a.T < 1 || a.T > (p.token_lanes ? 8 : 5) || p.wn < 1 || p.wk < 1 || W > 16) return (int)hipErrorInvalidValue;
  if (limb_lds_bytes(a.T, a.K, a.G, p) > (p.token_lanes || p.resident ? kLimbMaxLdsResident : kLimbMaxLds))
    return (int)hipErrorInvalidValue;
  if (p.token_lanes) {
    if (a.T > 8) return (int)hipErrorInvalidValue;
    return (int)(a.T <= 4 ? launch_limb_t<4>(a, p, st) : launch_limb_t<8>(a, p, st));
  }
  return (int)(a.T == 1 ? launch_limb_t<1>(a, p, st) : launch_limb_t<5>(a, p, st));
}

}  // namespace tern
