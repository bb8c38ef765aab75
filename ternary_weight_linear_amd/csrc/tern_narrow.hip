// tern_narrow.hip -- small_t / small_t_tiled kernel for narrow layers (fewer
// than 1024 strips of 16 outputs: o_proj 5120 -> 5120, down 17408 -> 5120)
// on gfx950.
//
// y[t][n] = sum_g s[n][g] * sum_{k in g} w[n][k] * x[t][k], w in {-1,0,+1},
// one fp16 scale per G weights along K ("NInfer sm_89 fork" article, section
// 9 item 2); T = 2..16 are the draft-verify rungs of the rung map ("NINFER
// ternary perf-tuning" notes, section 2), whose split-K gating by layer shape
// (section 5) this kernel serves.
//
// A narrow layer has too few strips to give every CU work, and its codes are
// few enough (7-23 MB) that the whole launch is mostly ramp and tail. So the
// work is cut into one workgroup per (block of W strips, K part), about one
// per CU, and each wave asks for all of its codes at once: the codes of its
// strip's K part (KMAX k-tiles at most, 1 KiB each) are requested in the
// prologue, before any arithmetic, so the HBM queue holds the whole layer
// from the start. The activation rows of the part (ROWS x nkt x 256 bf16, the
// MFMA A operand, rows past T read as zero) are loaded once per workgroup and
// kept in LDS; every wave's MFMAs read them from there.
//
// The Pk partial sums of a strip block are added inside the same launch:
// each workgroup stores its fp32 partials with device-coherent stores (they
// are written through to where every XCD reads them), waits for them to
// complete, and adds one to the block's arrival counter. The workgroup that
// takes the counter to Pk is the last of its block: it sets the counter back
// to zero and adds the Pk partials in ascending part order (so the sum is the
// same whichever part finished last), with device-coherent loads, and writes
// y. No workgroup waits for another, so nothing depends on workgroups being
// co-resident. The counters live at the start of the caller's workspace,
// must be zero when a workspace is first used, and are zero again after every
// launch.
//
// Arithmetic per k-tile is the activation-tiled kernel's (tern_tile.hip):
// the codes decode to bf16 {0, +-2.0} B operands of v_mfma_f32_16x16x32_bf16,
// each 128- or 64-wide group's exact fp32 sum is folded into the total with
// one fma by its scale, and y is half the total.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

constexpr int kAuxCoherent = 16;  // sc1: device-scope coherent access

// Waits for this wave's LDS operations, then the workgroup barrier, without
// the workgroup fence of __syncthreads(), which would also wait for every
// outstanding global load (the codes still in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  asm volatile("s_barrier" ::: "memory");
}

// Grid: Pk * nblocks workgroups, linear id L -> part L % Pk, strip block
// L / Pk (consecutive ids go to different XCDs, so with Pk = 8 each XCD reads
// one part's activation rows). Block: W waves, wave w owning strip
// block * W + w over the part's k-tiles [kt0, kt0 + nkt), nkt <= KMAX.
// Dynamic LDS: narrow_lds_bytes(): the activation rows (NQ * W chunks of
// 1 KiB) + 16 bytes.
// part: Pk * T * N floats; counters: nblocks ints.
template <int ROWS, int W, int GPT, int KMAX, int D>
__global__ void __launch_bounds__(64 * W) tern_narrow_kernel(
    const uint16_t* __restrict__ x, int T, int K, const u32x4* __restrict__ codes,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int N, float* __restrict__ part,
    int* __restrict__ counters, int Pk) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TILE = ROWS * 512;              // bytes of one k-tile of activation rows
  constexpr int CPT = ROWS / 2;                 // 1 KiB chunks per k-tile
  constexpr int NQ = (CPT * KMAX + W - 1) / W;  // chunks per wave
  constexpr int MPG = 8 / GPT;                  // MFMAs (32 k each) per scale group
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NS = N >> 4, KT = K >> 8;
  const int L = blockIdx.x;
  const int pk = L % Pk, sb = L / Pk;
  const int kt0 = (pk * KT) / Pk;
  const int nkt = ((pk + 1) * KT) / Pk - kt0;  // <= KMAX (checked by the launcher)
  const int strip = sb * W + wave;
  const bool has_strip = strip < NS;
  int* flag = (int*)(smem + NQ * W * 1024);

  // 1. Activation rows of the part into registers (chunk q = k-tile q / CPT,
  // 1 KiB piece q % CPT; lane l holds position 64 (q % CPT) + l of the tile:
  // row p / 32, chunk slot p % 32, global chunk slot ^ (row & 15)). Chunks
  // past the part read as zero; every wave loads and stores all NQ of its
  // chunks, so that no load is moved next to a conditional use.
  const rsrc_t xrs = make_rsrc(x, (uint32_t)T * K * 2);  // rows past T read as zero
  const int xso = __builtin_amdgcn_readfirstlane(kt0 * 512);
  u32x4 xv[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = j * W + wave;
    const int p = 64 * (q % CPT) + lane;
    const int t = p >> 5;
    const int cl = (p & 31) ^ (t & 15);
    const int off = q < CPT * nkt ? (t * K + cl * 8) * 2 + (q / CPT) * 512 : kOffPastEnd;
    xv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, xso, 0));
  }
  // the code requests must not move above the activation loads: the wait
  // before the LDS stores below counts on them being younger
  __builtin_amdgcn_sched_barrier(0);

  // 2. The code and scale loads of the wave's strip, k-tile by k-tile (the
  // order in which the k-tiles are waited for), k-tiles past nkt dropped:
  // all of them up front (D >= KMAX), or D ahead of the k-tile in use.
  const int sidx = has_strip ? strip : 0;
  const rsrc_t crs = make_rsrc(codes + (size_t)sidx * KT * 64, has_strip ? (uint32_t)KT * 1024 : 0u);
  const rsrc_t srs = make_rsrc(scales + (size_t)sidx * KT * 16 * GPT, has_strip ? (uint32_t)KT * 16 * GPT * 2 : 0u);
  const int cso = __builtin_amdgcn_readfirstlane(kt0 * 1024);
  const int sso = __builtin_amdgcn_readfirstlane(kt0 * 16 * GPT * 2);
  u32x4 P[KMAX];
  uint32_t sw[KMAX][GPT / 2];
  auto load_kt = [&](int i) {
    const bool v = i < nkt;
    P[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         crs, v ? lane * 16 + i * 1024 : kOffPastEnd, cso, kAuxNontemporal));
    const int sv = v ? (lane & 15) * GPT * 2 + i * 16 * GPT * 2 : kOffPastEnd;
    if (GPT == 2) {
      sw[i][0] = __builtin_amdgcn_raw_buffer_load_b32(srs, sv, sso, 0);
    } else {
      const auto s2 = __builtin_amdgcn_raw_buffer_load_b64(srs, sv, sso, 0);
      sw[i][0] = s2[0];
      sw[i][GPT / 2 - 1] = s2[1];
    }
  };
  constexpr int DD = D < KMAX ? D : KMAX;  // k-tiles requested before the first is used
#pragma unroll
  for (int i = 0; i < DD; ++i) {
    load_kt(i);
    __builtin_amdgcn_sched_barrier(0);
  }

  // 3. Activation rows to LDS (position 64 c + l of k-tile i at byte
  // i * TILE + c * 1024 + l * 16, i.e. chunk q at q * 1024; the LDS holds
  // NQ * W chunks), then the barrier.
#pragma unroll
  for (int j = 0; j < NQ; ++j)
    *(u32x4*)(smem + (size_t)(j * W + wave) * 1024 + lane * 16) = xv[j];
  lds_barrier();

  // 4. The k-tiles, as their codes arrive. Accumulator e of lane l is
  // C[token 4 (l >> 4) + e][row l & 15]; A rows past ROWS repeat earlier
  // rows and only feed discarded outputs.
  const int tr = lane & (ROWS - 1);
  const int g = lane >> 4;
  f32x4 total = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i + DD < KMAX) load_kt(i + DD);  // the ring: k-tile i + DD is requested before k-tile i is used
    __builtin_amdgcn_sched_barrier(0);
    if (i < nkt) {
      const char* row = smem + i * TILE + tr * 512;
      bf16x8 xa[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) xa[m] = *(const bf16x8*)(row + (((4 * m + g) ^ (tr & 15)) << 4));
      const uint4 Pi = uint4{P[i].x, P[i].y, P[i].z, P[i].w};
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mm = 0; mm < MPG; ++mm) {
          const int m = gi * MPG + mm;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m], weights_operand(Pi, m), acc, 0, 0, 0);
        }
        const uint32_t spair = sw[i][gi >> 1];
        const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
        total[0] = __builtin_fmaf(sc, acc[0], total[0]);
        total[1] = __builtin_fmaf(sc, acc[1], total[1]);
        total[2] = __builtin_fmaf(sc, acc[2], total[2]);
        total[3] = __builtin_fmaf(sc, acc[3], total[3]);
      }
    }
  }

  const int n = strip * 16 + (lane & 15);
  const int tq = 4 * g;
  if (Pk == 1) {
    if (has_strip) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (tq + e < T) y[(size_t)(tq + e) * N + n] = 0.5f * total[e];
    }
    return;
  }

  // 5. Partials of this part: device-coherent stores, then every wave waits
  // for its own, the barrier, and one arrival on the block's counter.
  {
    const rsrc_t prs = make_rsrc(part + (size_t)pk * T * N, (uint32_t)T * N * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool v = has_strip && tq + e < T;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(total[e]), prs,
                                            v ? ((tq + e) * N + n) * 4 : kOffPastEnd, 0, kAuxCoherent);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  lds_barrier();                  // ... and every other wave's
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(counters + sb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lds_barrier();
  if (*flag != Pk - 1) return;  // not the last part of this block to finish
  if (threadIdx.x == 0) __hip_atomic_store(counters + sb, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 6. Last part of the block: y = 0.5 * sum over parts in ascending order,
  // four outputs per thread, the parts requested 8 at a time.
  const int n0 = sb * W * 16;
  const int nb = min(W * 16, N - n0);  // outputs of this block (a multiple of 16)
  const rsrc_t ars = make_rsrc(part, (uint32_t)Pk * T * N * 4);
  for (int c = threadIdx.x; c < T * (nb >> 2); c += 64 * W) {
    const int t = c / (nb >> 2);
    const int o = n0 + 4 * (c % (nb >> 2));
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < Pk; p0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             ars, p0 + j < Pk ? (((p0 + j) * T + t) * N + o) * 4 : kOffPastEnd,
                                             0, kAuxCoherent));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (p0 + j < Pk) sum += v[j];
    }
    *(f32x4*)(y + (size_t)t * N + o) = sum * 0.5f;
  }
}

template <int ROWS, int W, int GPT>
hipError_t launch_narrow_k(const SmallTArgs& a, const NarrowPlan& p, float* part, int* counters,
                           hipStream_t st) {
  const size_t lds = (size_t)narrow_lds_bytes(p);
  dim3 grid((unsigned)(p.strip_blocks * p.k_parts)), block(64 * W);
  switch (p.kmax) {
#define TERN_NARROW_LAUNCH(KM)                                                                          \
  case KM:                                                                                             \
    if constexpr (W * KM <= 192) { /* 16 waves: 128 VGPRs each, at most 12 k-tiles of codes */        \
      if (p.depth == 4)                                                                                \
        hipLaunchKernelGGL((tern_narrow_kernel<ROWS, W, GPT, KM, 4>), grid, block, lds, st, a.x, a.T,  \
                           a.K, (const u32x4*)a.codes, a.scales, a.y, a.N, part, counters, p.k_parts); \
      else                                                                                             \
        hipLaunchKernelGGL((tern_narrow_kernel<ROWS, W, GPT, KM, 16>), grid, block, lds, st, a.x, a.T, \
                           a.K, (const u32x4*)a.codes, a.scales, a.y, a.N, part, counters, p.k_parts); \
    } else {                                                                                           \
      return hipErrorInvalidValue;                                                                     \
    }                                                                                                  \
    break;
    TERN_NARROW_LAUNCH(4)
    TERN_NARROW_LAUNCH(8)
    TERN_NARROW_LAUNCH(12)
    TERN_NARROW_LAUNCH(16)
#undef TERN_NARROW_LAUNCH
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int ROWS, int W>
hipError_t launch_narrow_w(const SmallTArgs& a, const NarrowPlan& p, float* part, int* counters,
                           hipStream_t st) {
  return a.G == 128 ? launch_narrow_k<ROWS, W, 2>(a, p, part, counters, st)
                    : launch_narrow_k<ROWS, W, 4>(a, p, part, counters, st);
}

template <int ROWS>
hipError_t launch_narrow_r(const SmallTArgs& a, const NarrowPlan& p, float* part, int* counters,
                           hipStream_t st) {
  switch (p.waves) {
    case 8: return launch_narrow_w<ROWS, 8>(a, p, part, counters, st);
    case 16: return launch_narrow_w<ROWS, 16>(a, p, part, counters, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t narrow_partial_bytes(const NarrowPlan& p, int T, int N) {
  return p.k_parts > 1 ? (size_t)p.k_parts * T * N * sizeof(float) : 0;
}

int narrow_lds_bytes(const NarrowPlan& p) {
  const int chunks = p.rows / 2 * p.kmax;                      // 1 KiB chunks of activation rows
  return (chunks + p.waves - 1) / p.waves * p.waves * 1024 + 16;  // NQ * W of them, + the flag
}

int launch_narrow(const SmallTArgs& a, const NarrowPlan& p, void* part, int* counters, void* stream) {
  const int NS = a.N / 16, KT = a.K / 256;
  if (a.T < 1 || a.T > p.rows || p.strip_blocks != (NS + p.waves - 1) / p.waves || p.k_parts < 1 ||
      (p.depth != 0 && p.depth != 4) ||
      p.k_parts > KT || (p.k_parts > 1 && (!part || !counters)))
    return (int)hipErrorInvalidValue;
  // every part's k-tiles fit the register ring: ceil(KT / Pk) <= kmax
  if ((KT + p.k_parts - 1) / p.k_parts > p.kmax) return (int)hipErrorInvalidValue;
  if ((long)p.strip_blocks * p.k_parts > 65535L * 64) return (int)hipErrorInvalidValue;
  // partial offsets are 32-bit byte offsets
  if ((size_t)p.k_parts * a.T * a.N * sizeof(float) >= (size_t)1 << 31) return (int)hipErrorInvalidValue;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (p.rows) {
    case 4: e = launch_narrow_r<4>(a, p, (float*)part, counters, st); break;
    case 8: e = launch_narrow_r<8>(a, p, (float*)part, counters, st); break;
    case 16: e = launch_narrow_r<16>(a, p, (float*)part, counters, st); break;
    default: return (int)hipErrorInvalidValue;
  }
  return kernel_launched((int)e, TERN_KERNEL_SMALLT_NARROW);
}

}  // namespace tern
