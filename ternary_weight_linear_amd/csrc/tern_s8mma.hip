// tern_s8mma.hip -- the s8 rung's contraction for activations quantised in
// the operand order (include/tern.h, TERN_Q_OPERAND_ORDER): int8 activations
// x ternary weights on v_mfma_i32_16x16x64_i8, fp32 scale epilogue.
//
// y[t][n] = scale_t * sum_g s[n][g] * acc[t][n][g], acc = sum_{k in g} q[t][k] * w[n][k]
// ("NInfer sm_89 fork" article, sections 7 and 9 item 2: prefill activations
// quantised per token to int8, the product an integer contraction).
//
// Cost model on MI355X. Per 16x16 output tile and 128-wide scale group the
// matrix core runs 2 MFMAs (32 cycles) and the vector ALU converts and scales
// 4 accumulators per lane (8 instructions, about the same time); measured on
// the part, the two units hardly overlap, so the kernel spends as little ALU
// time per MFMA as it can:
//  * wave tile TB x 16 tokens by S x 16 outputs (TB token blocks, S strips):
//    each decoded weight operand feeds TB MFMAs, each A fragment S MFMAs;
//  * the codes decode straight into int8 B operands, (word << 2i) &
//    0xC0C0C0C0 = 64*w (weights_operand_i8), so the totals carry a factor 64:
//    fma(float(64*acc), s, 64*total) = 64 * fma(acc, s, total) exactly (every
//    term is a multiple of 2^-24, so nothing is subnormal), and the fp16 scale
//    feeds the fma directly (v_fma_mix_f32, no conversion);
//  * the epilogue per group and accumulator is one convert and one fma, in
//    ascending group order, then y = (total * 2^-6) * scale_t, bit-identical
//    to summing acc * s and multiplying by scale_t.
// Workgroup: 4 waves share one TB x 16-token activation tile in LDS (double
// buffered, filled by direct buffer-to-LDS loads; the 16-byte chunks of row r
// sit at chunk ^ (r & 15) so that the 16 rows of a fragment read hits 16
// different banks) and take S strips each.
// Tile order: workgroups go to the 8 XCDs round-robin. When the token tiles
// split evenly over the XCDs, each XCD takes its own token tiles with the
// token tile fastest, so each code block is fetched into its L2 once and
// shared by the workgroups it runs together.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

template <int GPT, int S>
struct S8mStage {
  u32x4 code[S];            // the lane's 16 code bytes of each strip
  uint32_t sw[S][GPT / 2];  // fp16 scale pairs of row (lane & 15)
};

// The workgroup's side of a k-tile handoff in the D-deep pipeline: wait until
// at most N of this wave's loads are outstanding (they retire in order), then
// the barrier, without the workgroup fence of __syncthreads() (that fence
// would wait for every outstanding buffer-to-LDS load and throw the lead
// away). The "memory" clobber keeps the compiler from moving loads or LDS
// reads across it.
template <int N>
__device__ __forceinline__ void s8m_handoff() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  asm volatile("s_barrier" ::: "memory");
}

// D: k-tiles in flight. D = 2 is the double-buffered pipeline of the
// compute-bound shapes; D = 4 keeps three k-tiles of activations and codes in
// flight for the short, memory-bound prefills. gridDim.y = Pk splits the
// k-tiles over workgroups (Pk > 1: fp32 partial totals to part[Pk][T][N],
// added by tern_s8m_reduce_kernel).
template <int GPT, int TB, int S, int D, bool DEBUG_ACC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) tern_s8m_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ act_scale, int T, int K,
    const u32x4* __restrict__ codes, const uint16_t* __restrict__ scales, float* __restrict__ y,
    int32_t* __restrict__ acc_out, int N, int nx, int ny, int xrows, float* __restrict__ part) {
  constexpr int BM = 16 * TB;    // tokens per tile
  constexpr int KBPG = 4 / GPT;  // 64-wide k-blocks per scale group
  constexpr int kS8WgStrips = 4 * S;
  static_assert(D == 2 || D == 4, "pipeline depth");
  static_assert(!DEBUG_ACC || D == 2, "the accumulator export uses the double-buffered pipeline");
  __shared__ __attribute__((aligned(1024))) int8_t As[D][BM * 256];

  // Tile (ty, tx) of this workgroup. xrows == 0: plain order, output blocks
  // fastest. xrows > 0 (ny == 8 * xrows): block b runs on XCD b % 8 as its
  // (b / 8)-th block there, and XCD x takes token tiles [x * xrows, (x + 1) *
  // xrows) with the token tile fastest: the workgroups it runs together share
  // each code block, and its few activation tiles stay in its L2.
  int ty, tx;
  if (xrows) {
    const int xcd = (int)(blockIdx.x & 7), slot = (int)(blockIdx.x >> 3);
    ty = xcd * xrows + slot % xrows;
    tx = slot / xrows;
  } else {
    ty = (int)blockIdx.x / nx;
    tx = (int)blockIdx.x - ty * nx;
  }
  const int tile = ty * nx + tx;
  if (tile >= nx * ny) return;  // uniform over the workgroup (never taken: the grid is nx * ny)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int NS = N >> 4, KT = K >> 8, NG = K / (256 / GPT);
  const int Pk = gridDim.y, pk = blockIdx.y;
  const int kt0 = (pk * KT) / Pk;
  const int nkt = ((pk + 1) * KT) / Pk - kt0;  // >= 1: Pk <= KT
  const int t0 = ty * BM;
  const int nt = min(BM, T - t0);
  const int st0 = tx * kS8WgStrips + wave * S;  // first strip of this wave
  const int nst = max(0, min(S, NS - st0));     // of which exist

  // The tile's token scales, read once here and kept in LDS for the
  // epilogue: a load per output row at the end would wait for every store
  // issued before it (the vector memory counter covers both), one memory
  // round trip per row.
  __shared__ float sas[BM];
  const bool stage_scales = !DEBUG_ACC && Pk == 1;
  float as_ld = 0.f;
  if (stage_scales && tid < BM) as_ld = act_scale[t0 + min(tid, nt - 1)];

  const rsrc_t qr = make_rsrc(q + (size_t)t0 * K, (uint32_t)nt * K);
  const rsrc_t cr = make_rsrc(codes + (size_t)min(st0, NS) * KT * 64, (uint32_t)nst * KT * 1024);
  const rsrc_t sr = make_rsrc(scales + (size_t)min(st0, NS) * KT * 16 * GPT,
                              (uint32_t)nst * KT * 16 * GPT * 2);

  // Activation tile kt into buffer buf: BM rows of 256 bytes, 4 rows per
  // direct-to-LDS load (64 lanes x 16 bytes); wave w loads rows
  // [w*4*TB, (w+1)*4*TB). Lane i of a load writes LDS chunk i % 16 of row
  // base + i / 16 and fetches the row's global chunk (i % 16) ^ (row & 15).
  // Rows past the last token read as zeros (buffer range check).
  auto stage_a = [&](int kt, int buf) {
    kt = __builtin_amdgcn_readfirstlane(kt);
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int rbase = wave * 4 * TB + 4 * j;
      const int row = rbase + (lane >> 4);
      const int chunk = (lane & 15) ^ (row & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qr, (__attribute__((address_space(3))) void*)&As[buf][rbase * 256], 16, row * K + chunk * 16,
          kt * 256, 0, 0);  // cached: every workgroup of this token tile on the XCD reads it
    }
  };
  auto load_w = [&](int kt, S8mStage<GPT, S>& b) {
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

  // One k-tile: per scale group, the A fragments of its k-blocks (shared by
  // both strips), then per strip KBPG x TB MFMAs and the group's epilogue.
  auto compute = [&](int kt, int buf, const S8mStage<GPT, S>& b) {
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      i32x4 af[KBPG][TB];
#pragma unroll
      for (int kk = 0; kk < KBPG; ++kk)
#pragma unroll
        for (int a = 0; a < TB; ++a) {
          const int chunk = (4 * (gi * KBPG + kk) + g) ^ r;  // row & 15 == r
          af[kk][a] = *(const i32x4*)&As[buf][(a * 16 + r) * 256 + chunk * 16];
        }
      const int gidx = kt * GPT + gi;
#pragma unroll
      for (int c = 0; c < S; ++c) {
        i32x4 acc[TB];
#pragma unroll
        for (int kk = 0; kk < KBPG; ++kk) {
          const i32x4 bf = weights_operand_i8(b.code[c][gi * KBPG + kk]);
#pragma unroll
          for (int a = 0; a < TB; ++a)
            acc[a] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[kk][a], bf,
                                                           kk == 0 ? i32x4{0, 0, 0, 0} : acc[a], 0, 0, 0);
        }
        if (DEBUG_ACC) {
          const int n = (st0 + c) * 16 + r;  // accumulator column of this lane
#pragma unroll
          for (int a = 0; a < TB; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int tl = a * 16 + 4 * g + e;
              if (tl < nt && c < nst) acc_out[((size_t)(t0 + tl) * N + n) * NG + gidx] = acc[a][e] >> 6;
            }
        } else {
          const uint32_t sp = b.sw[c][gi >> 1];
          const float sv = half_bits_to_float((uint16_t)((gi & 1) ? (sp >> 16) : (sp & 0xffffu)));
#pragma unroll
          for (int a = 0; a < TB; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) tot[a][c][e] = __builtin_fmaf((float)acc[a][e], sv, tot[a][c][e]);
        }
      }
    }
  };

  // The same k-tile as a software pipeline (not DEBUG_ACC). Unit u = (group
  // gi, strip c) runs its KBPG * TB MFMAs while the vector ALU folds the
  // previous unit's accumulators into the totals and decodes the next unit's
  // weight operands: independent instructions, which the matrix core and the
  // vector ALU execute side by side when they are interleaved (measured on
  // the part: 8 i8 MFMAs with 16 independent VALU instructions in between
  // take about the time of the MFMAs alone; done one after the other, the
  // sum of both). The previous unit of a k-tile's first unit is the last of
  // the k-tile before (strip S - 1, across the barrier); pend starts as zeros
  // with a zero scale, whose fold adds +0 to a +0 total. Per strip the folds
  // still run in ascending group order, so the totals are those of compute.
  i32x4 pend[TB];
  float pend_s = 0.f;
#pragma unroll
  for (int a = 0; a < TB; ++a) pend[a] = i32x4{0, 0, 0, 0};
  constexpr int kValuPerMfma = (8 * TB + 7 * KBPG + 2 + KBPG * TB - 1) / (KBPG * TB);
  auto compute_p = [&](int kt, int buf, const S8mStage<GPT, S>& b) {
    (void)kt;
    i32x4 bq[KBPG];
#pragma unroll
    for (int kk = 0; kk < KBPG; ++kk) bq[kk] = weights_operand_i8(b.code[0][kk]);
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      i32x4 af[KBPG][TB];
#pragma unroll
      for (int kk = 0; kk < KBPG; ++kk)
#pragma unroll
        for (int a = 0; a < TB; ++a) {
          const int chunk = (4 * (gi * KBPG + kk) + g) ^ r;  // row & 15 == r
          af[kk][a] = *(const i32x4*)&As[buf][(a * 16 + r) * 256 + chunk * 16];
        }
#pragma unroll
      for (int c = 0; c < S; ++c) {
        i32x4 acc[TB];
#pragma unroll
        for (int kk = 0; kk < KBPG; ++kk)
#pragma unroll
          for (int a = 0; a < TB; ++a)
            acc[a] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[kk][a], bq[kk],
                                                           kk == 0 ? i32x4{0, 0, 0, 0} : acc[a], 0, 0, 0);
        // the next unit's weight operands, inside this k-tile
        const int cn = c + 1 < S ? c + 1 : 0;
        const int gn = c + 1 < S ? gi : gi + 1;
        if (gn < GPT) {
#pragma unroll
          for (int kk = 0; kk < KBPG; ++kk) bq[kk] = weights_operand_i8(b.code[cn][gn * KBPG + kk]);
        }
        // the previous unit's epilogue
        const int cp = c == 0 ? S - 1 : c - 1;
#pragma unroll
        for (int a = 0; a < TB; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) tot[a][cp][e] = __builtin_fmaf((float)pend[a][e], pend_s, tot[a][cp][e]);
        const uint32_t sp = b.sw[c][gi >> 1];
        pend_s = half_bits_to_float((uint16_t)((gi & 1) ? (sp >> 16) : (sp & 0xffffu)));
#pragma unroll
        for (int a = 0; a < TB; ++a) pend[a] = acc[a];
#pragma unroll
        for (int m = 0; m < KBPG * TB; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // then vector ALU work
        }
      }
    }
  };
  // Folds the last pending unit (strip S - 1) after the final k-tile.
  auto flush = [&]() {
#pragma unroll
    for (int a = 0; a < TB; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[a][S - 1][e] = __builtin_fmaf((float)pend[a][e], pend_s, tot[a][S - 1][e]);
  };
  auto run = [&](int kt, int buf, const S8mStage<GPT, S>& b) {
    if constexpr (DEBUG_ACC)
      compute(kt, buf, b);
    else
      compute_p(kt, buf, b);
  };

  if constexpr (D == 2) {
    // Pipeline, one barrier per k-tile: the activation tile and the codes of
    // k-tile kt+1 are requested before the MFMAs of k-tile kt; then each wave
    // waits for its loads and meets the others at the barrier, after which
    // tile kt+1 is complete in LDS and nobody reads tile kt's buffer any more.
    // The loop runs k-tiles in pairs (buffers 0 then 1) with no exit in
    // between, so the totals keep their registers; with an even tile count the
    // last pair re-requests the last tile, with an odd one the tail computes
    // it from buffer 0.
    const int klast = kt0 + nkt - 1;
    S8mStage<GPT, S> wA, wB;
    stage_a(kt0, 0);
    load_w(kt0, wA);
    if (stage_scales && tid < BM) sas[tid] = as_ld;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int kt = kt0;
    for (; kt + 2 <= kt0 + nkt; kt += 2) {
      stage_a(kt + 1, 1);
      load_w(kt + 1, wB);
      __builtin_amdgcn_sched_barrier(0);
      run(kt, 0, wA);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const int k2 = min(kt + 2, klast);
      stage_a(k2, 0);
      load_w(k2, wA);
      __builtin_amdgcn_sched_barrier(0);
      run(kt + 1, 1, wB);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (kt <= klast) run(kt, 0, wA);
  } else {
    // Ring of D buffers: k-tile i sits in activation buffer i % D and code
    // stage i % D (i counted from kt0). Iteration i requests k-tile i + D - 1
    // (clamped to the last one, so every iteration issues the same TB + 2S
    // loads per wave) into the buffer of k-tile i - 1, which every wave
    // finished before the previous barrier, computes k-tile i, and hands over
    // k-tile i + 1: at most (D - 2) iterations of loads may stay outstanding.
    constexpr int L = TB + 2 * S;  // loads per wave per k-tile
    S8mStage<GPT, S> ring[D];
#pragma unroll
    for (int j = 0; j < D - 1; ++j) {
      const int kn = kt0 + min(j, nkt - 1);
      stage_a(kn, j);
      load_w(kn, ring[j]);
    }
    if (stage_scales && tid < BM) sas[tid] = as_ld;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // LDS writes done (lgkmcnt 0; vmcnt, expcnt free)
    s8m_handoff<(D - 2) * L>();
    int i = 0;
    for (; i + D <= nkt; i += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int kn = kt0 + min(i + j + D - 1, nkt - 1);
        stage_a(kn, (j + D - 1) % D);
        load_w(kn, ring[(j + D - 1) % D]);
        __builtin_amdgcn_sched_barrier(0);
        run(kt0 + i + j, j, ring[j]);
        s8m_handoff<(D - 2) * L>();
      }
    }
    // Tail: fewer than D k-tiles left, all requested already; k-tile i is in
    // place, the others are waited for one by one.
#pragma unroll
    for (int j = 0; j < D - 1; ++j) {
      if (i + j < nkt) {  // uniform over the workgroup
        if (j > 0) s8m_handoff<0>();
        run(kt0 + i + j, j, ring[j]);
      }
    }
  }
  if constexpr (!DEBUG_ACC) flush();

  if (!DEBUG_ACC && Pk > 1) {
    // Partial totals of this K part, 2^-6 taken out; the reduce kernel adds
    // the parts in ascending order and applies the token scales.
    float* mine = part + (size_t)pk * T * N;
#pragma unroll
    for (int a = 0; a < TB; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tl = a * 16 + 4 * g + e;
        if (tl >= nt) continue;
#pragma unroll
        for (int c = 0; c < S; ++c)
          if (c < nst) mine[(size_t)(t0 + tl) * N + (st0 + c) * 16 + r] = tot[a][c][e] * 0.015625f;
      }
    return;
  }
  if (!DEBUG_ACC) {
#pragma unroll
    for (int a = 0; a < TB; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tl = a * 16 + 4 * g + e;
        if (tl >= nt) continue;
        const float as = sas[tl];
#pragma unroll
        for (int c = 0; c < S; ++c)
          if (c < nst) y[(size_t)(t0 + tl) * N + (st0 + c) * 16 + r] = (tot[a][c][e] * 0.015625f) * as;
      }
  }
}

// y[t][n] = act_scale[t] * sum_{p < Pk} part[p][t][n], parts in ascending
// order; four outputs per thread, token t = blockIdx.y. The parts are
// requested 8 at a time before they are added (each is a memory round trip:
// they were just written on other XCDs).
__global__ void __launch_bounds__(256) tern_s8m_reduce_kernel(const float* __restrict__ part,
                                                             const float* __restrict__ act_scale,
                                                             float* __restrict__ y, int T, int N, int Pk) {
  const int n4 = N >> 2;
  const int c = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  const int t = (int)blockIdx.y;
  if (c >= n4) return;
  const size_t i = (size_t)t * n4 + c;
  const f32x4* src = (const f32x4*)part + i;
  const size_t stride = (size_t)T * n4;
  // -0 + v == v for every v (zeros keep their sign): the sum starts as part 0
  f32x4 sum = f32x4{-0.f, -0.f, -0.f, -0.f};
  for (int p0 = 0; p0 < Pk; p0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (p0 + j < Pk) v[j] = __builtin_nontemporal_load(src + (size_t)(p0 + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (p0 + j < Pk) sum += v[j];
  }
  ((f32x4*)y)[i] = sum * act_scale[t];
}

template <int GPT, int TB, int S, int D, bool DEBUG_ACC>
hipError_t launch_s8m_t(const S8Args& a, const S8Plan& p, float* part, hipStream_t st) {
  constexpr int kS8WgStrips = 4 * S;
  const int NS = a.N / 16;
  const int nx = (NS + kS8WgStrips - 1) / kS8WgStrips;
  const int ny = (a.T + 16 * TB - 1) / (16 * TB);
  const int xrows = (p.xcd_order && ny % 8 == 0) ? ny / 8 : 0;
  hipLaunchKernelGGL((tern_s8m_kernel<GPT, TB, S, D, DEBUG_ACC>), dim3(nx * ny, p.k_parts), dim3(256), 0,
                     st, a.q, a.act_scale, a.T, a.K, (const u32x4*)a.codes, a.scales, a.y, a.acc_out,
                     a.N, nx, ny, xrows, part);
  return (hipError_t)kernel_launched((int)hipGetLastError(),
                                     DEBUG_ACC ? TERN_KERNEL_S8_ACC_EXPORT : TERN_KERNEL_S8_MMA);
}

template <int GPT, int TB, int S, bool DEBUG_ACC>
hipError_t launch_s8m_d(const S8Args& a, const S8Plan& p, float* part, hipStream_t st) {
  if constexpr (DEBUG_ACC && TB * S >= 16) {
    // the accumulator export at 64 x 64 would spill: tern_debug_s8_acc runs
    // that tile as 64 x 32
    return hipErrorInvalidValue;
  } else if constexpr (DEBUG_ACC || TB * S >= 16 || (TB == 2 && S == 4)) {
    // (the 64 x 64 and 32 x 64 wave tiles have no registers left for two more
    // code stages)
    return launch_s8m_t<GPT, TB, S, 2, DEBUG_ACC>(a, p, part, st);
  } else {
    return p.depth == 4 ? launch_s8m_t<GPT, TB, S, 4, false>(a, p, part, st)
                        : launch_s8m_t<GPT, TB, S, 2, false>(a, p, part, st);
  }
}

template <int GPT, bool DEBUG_ACC>
hipError_t launch_s8m_g(const S8Args& a, const S8Plan& p, float* part, hipStream_t st) {
  switch (p.token_blocks * 16 + p.strips) {
    case 2 * 16 + 1: return launch_s8m_d<GPT, 2, 1, DEBUG_ACC>(a, p, part, st);
    case 3 * 16 + 1: return launch_s8m_d<GPT, 3, 1, DEBUG_ACC>(a, p, part, st);
    case 4 * 16 + 1: return launch_s8m_d<GPT, 4, 1, DEBUG_ACC>(a, p, part, st);
    case 2 * 16 + 2: return launch_s8m_d<GPT, 2, 2, DEBUG_ACC>(a, p, part, st);
    case 2 * 16 + 4: return launch_s8m_d<GPT, 2, 4, DEBUG_ACC>(a, p, part, st);
    case 4 * 16 + 2: return launch_s8m_d<GPT, 4, 2, DEBUG_ACC>(a, p, part, st);
    case 4 * 16 + 4: return launch_s8m_d<GPT, 4, 4, DEBUG_ACC>(a, p, part, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int launch_s8_operand_order(const S8Args& a, const S8Plan& p, void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool dbg = a.acc_out != nullptr;
  if (p.k_parts < 1 || p.k_parts > a.K / 256 || (p.depth != 2 && p.depth != 4)) return (int)hipErrorInvalidValue;
  if (p.k_parts > 1 && (dbg || ws == nullptr || a.N % 4 != 0 || a.T > 65535)) return (int)hipErrorInvalidValue;
  float* part = p.k_parts > 1 ? (float*)ws : nullptr;
  hipError_t e;
  if (a.G == 128)
    e = dbg ? launch_s8m_g<2, true>(a, p, part, st) : launch_s8m_g<2, false>(a, p, part, st);
  else
    e = dbg ? launch_s8m_g<4, true>(a, p, part, st) : launch_s8m_g<4, false>(a, p, part, st);
  if (e != hipSuccess || p.k_parts == 1) return (int)e;
  hipLaunchKernelGGL(tern_s8m_reduce_kernel, dim3((unsigned)((a.N / 4 + 255) / 256), (unsigned)a.T), dim3(256), 0,
                     st, (const float*)part, a.act_scale, a.y, a.T, a.N, p.k_parts);
  return kernel_launched((int)hipGetLastError(), TERN_KERNEL_S8_REDUCE);
}

size_t s8_partial_bytes(const S8Plan& p, int T, int N) {
  return p.k_parts > 1 ? (size_t)p.k_parts * T * N * sizeof(float) : 0;
}

}  // namespace tern
