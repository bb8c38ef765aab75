// tern_chain.hip -- a whole decode pass (T = 1) over a chain of ternary
// projections in one launch, for the per-launch ramp and tail of short
// matrices: the pages replay each decode round as one captured graph of
// about 1224 kernels ("NINFER ternary perf-tuning" notes, section 6; "NInfer
// sm_89 fork" article, section 9 item 5), where every launch pays its own
// ramp and drain.
//
// One workgroup of 12 waves per CU, launched cooperatively (all resident or
// the launch fails). Each projection's 16-row strips are cut into units of
// wn strips (the gemv's plan, K split over wk waves). The host gives every
// workgroup a list of units in projection order, balanced between the
// waits (each unit to the least loaded workgroup, by its bytes of codes and
// its K); every workgroup walks the projections in order. A projection may depend on earlier ones
// (after = j: items 0..j all finished): a workgroup requests its unit's
// first k-tiles of codes, which do not depend on anything, and only then
// waits, so the weight stream goes on while the previous projection drains.
//
// Completion: after its units of a projection that a later one waits on,
// every workgroup (with or without units) makes its stores visible at
// device scope (release fence) and adds one to the projection's counter;
// waiting for items 0..j means waiting for counter j to reach the number of
// workgroups, then an acquire fence. Each wait polls at most spin_limit
// times; on giving up it sets *error_flag and the workgroup skips the rest
// of the chain, so every wave exits. The last workgroup out zeroes the
// counters for the next launch.
//
// The arithmetic of a unit is the T = 1 integer-limb gemv of tern_limb.hip
// (limbs of x in LDS, codes decoded into i8 MFMA operands, per-group fp32
// epilogue, K shares added in ascending order), so y is bit-identical to
// tern_linear's gemv rung for the same weights.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

constexpr int kChainThreads = 64 * kChainWaves;
constexpr int kChainDepth = 4;  // k-tiles of codes in flight per wave

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // finite inputs
}

template <int GPT>
__global__ void __launch_bounds__(kChainThreads) tern_chain_kernel(const ChainEntry* __restrict__ table,
                                                                   int count, const int* __restrict__ wg_begin,
                                                                   const int2* __restrict__ work,
                                                                   int* __restrict__ counters,
                                                                   int* __restrict__ error_flag, int spin_limit) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_abort;
  constexpr int KBPG = 4 / GPT;
  constexpr int D = kChainDepth;
  const int P = gridDim.x, b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  if (tid == 0) s_abort = 0;
  __syncthreads();
  int wp = wg_begin[b];             // this workgroup's work list: (projection, unit) pairs,
  const int wend = wg_begin[b + 1];  // in projection order
  int prepped = -1;                  // projection whose limbs of x are in LDS

  for (int i = 0; i < count && !s_abort; ++i) {
    const ChainEntry e = table[i];
    const int NS = e.n >> 4, K = e.k, KT = K >> 8;
    const int Wn = e.wn, Wk = e.wk;
    const int wn = wave % Wn, wk = wave / Wn;
    const int rs = K + 64;
    int* dexp = (int*)(smem + (size_t)3 * rs);
    char* lsc = smem + (size_t)3 * rs + (size_t)KT * 4;  // [Wn][KT][16][GPT] fp16
    float* red = (float*)(lsc + (size_t)Wn * KT * 16 * GPT * 2);  // [Wk][Wn][16]: after the limbs and scales
    bool waited = e.after < 0;
    for (; wp < wend && work[wp].x == i; ++wp) {
      const int u = work[wp].y;
      const int strip = u * Wn + wn;
      const bool has = wk < Wk && strip < NS;
      const int kt0 = has ? (wk * KT) / Wk : 0;
      const int nkt = has ? ((wk + 1) * KT) / Wk - kt0 : 0;
      const rsrc_t crs = make_rsrc((const char*)e.codes + (size_t)(has ? strip : 0) * KT * 1024,
                                   has ? (uint32_t)KT * 1024 : 0u);
      auto load = [&](u32x4& P4, int j) {
        const int kt = __builtin_amdgcn_readfirstlane(min(kt0 + j, KT - 1));
        const int cv = j < nkt ? lane * 16 : kOffPastEnd;
        P4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, cv, kt * 1024, kAuxNontemporal));
      };
      // 1. the first k-tiles of codes: they depend on nothing
      u32x4 ring[D];
#pragma unroll
      for (int j = 0; j < D - 1; ++j) load(ring[j], j);

      // 2. the dependency, once per projection and workgroup
      if (!waited) {
        if (tid == 0) {
          bool ok = false;
          for (int it = 0;; ++it) {
            if (__hip_atomic_load(&counters[e.after], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= P) {
              ok = true;
              break;
            }
            if (__hip_atomic_load(error_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
            if (it >= spin_limit) {
              __hip_atomic_store(error_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // later reads of x see the producers' stores
          if (!ok) s_abort = 1;
        }
        waited = true;
      }
      __syncthreads();  // the wait, and the previous unit's last reads of the LDS
      if (s_abort) break;

      // 3. limbs of x (unless this workgroup's previous unit was of the same
      //    projection: they are still in LDS) and the unit's scales into LDS
      //    (as the gemv kernel)
      const rsrc_t xr = make_rsrc(e.x, (uint32_t)K * 2);
      const int nchunk = prepped == i ? 0 : K >> 4;
      prepped = i;
      for (int c = tid; c < nchunk; c += kChainThreads) {  // rows of 16 lanes are wholly in or out
        const int base = 64 * (c >> 2) + 8 * (c & 3);
        const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, base * 2, 0, 0));
        const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (base + 32) * 2, 0, 0));
        const int d = limb_shift(row16_max_u32(absmax16(lo, hi)));
        u32x4 o0, o1, o2;
        limb_chunk(lo, hi, d, o0, o1, o2);
        char* row = smem + 16 * c;
        *(u32x4*)row = o0;
        *(u32x4*)(row + rs) = o1;
        *(u32x4*)(row + 2 * rs) = o2;
        if ((c & 15) == 0) dexp[c >> 4] = d;
      }
      const int nsb = min(Wn, NS - u * Wn);
      const int nsc = nsb * KT * 2 * GPT;  // 16-byte chunks of scales
      const rsrc_t wsr = make_rsrc(e.scales + (size_t)u * Wn * KT * 16 * GPT, (uint32_t)nsc * 16);
      for (int c = tid; c < nsc; c += kChainThreads)
        *(u32x4*)(lsc + 16 * c) = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wsr, c * 16, 0, 0));
      __syncthreads();

      // 4. the contraction over this wave's k-tiles
      float total = 0.f;
      const char* abase = smem + (size_t)(r < 3 ? r : 0) * rs + 16 * g;
      const char* wsc = lsc + ((size_t)wn * KT * 16 + r) * GPT * 2;
      auto compute = [&](const u32x4& P4, int j) {
        const int kt = kt0 + j;
        i32x4 a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = *(const i32x4*)(abase + 64 * (4 * kt + q));
        const int dsh = dexp[kt] - 6;
        uint32_t sw[GPT / 2];
        const char* sp = wsc + (size_t)kt * 16 * GPT * 2;
        if (GPT == 2) {
          sw[0] = *(const uint32_t*)sp;
        } else {
          const uint2 v = *(const uint2*)sp;
          sw[0] = v.x;
          sw[GPT / 2 - 1] = v.y;
        }
        float part = 0.f;
#pragma unroll
        for (int gi = 0; gi < GPT; ++gi) {
          i32x4 acc = i32x4{0, 0, 0, 0};
#pragma unroll
          for (int kk = 0; kk < KBPG; ++kk) {
            const int q = gi * KBPG + kk;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[q], weights_operand_i8(P4[q]), acc, 0, 0, 0);
          }
          const uint32_t spair = sw[gi >> 1];
          const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
          const int low = (int)(((uint32_t)acc[1] << 8) + (uint32_t)acc[0]);  // 256 a1 + a0
          const float v = __builtin_fmaf(65536.0f, (float)acc[2], (float)low);
          part = gi == 0 ? sc * v : __builtin_fmaf(sc, v, part);
        }
        total += __builtin_ldexpf(part, dsh);
      };
      int j = 0;
      for (; j + D <= nkt; j += D) {
#pragma unroll
        for (int jj = 0; jj < D; ++jj) {
          load(ring[(jj + D - 1) % D], j + jj + D - 1);
          __builtin_amdgcn_sched_barrier(0);
          compute(ring[jj], j + jj);
        }
      }
#pragma unroll
      for (int jj = 0; jj < D - 1; ++jj)
        if (j + jj < nkt) compute(ring[jj], j + jj);

      // 5. y (and its bf16 copy); K shares added through LDS in ascending order
      if (Wk == 1) {
        if (has && lane < 16) {
          e.y[(size_t)strip * 16 + lane] = total;
          if (e.y_bf16) e.y_bf16[(size_t)strip * 16 + lane] = f32_to_bf16_rne(total);
        }
      } else {
        __syncthreads();  // the previous unit's readers of red are done
        if (wk < Wk && lane < 16) red[(wk * Wn + wn) * 16 + lane] = total;
        __syncthreads();
        if (tid < nsb * 16) {
          const int ls = tid >> 4, col = tid & 15;
          float sum = 0.f;
          for (int w = 0; w < Wk; ++w) sum += red[(w * Wn + ls) * 16 + col];
          const size_t o = (size_t)(u * Wn + ls) * 16 + col;
          e.y[o] = sum;
          if (e.y_bf16) e.y_bf16[o] = f32_to_bf16_rne(sum);
        }
      }
    }
    if (s_abort) break;
    // 6. this workgroup is done with projection i (and, in order, with all
    //    before it): count it for the projections that wait
    if (e.signal) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed (reached its L2)
      __syncthreads();                // ... and every other wave's
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // write them back for every XCD
        __hip_atomic_fetch_add(&counters[i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // 7. the last workgroup out zeroes the counters for the next launch. No
  //    data is published here (the kernel's end does that), so no release
  //    fence (an L2 write-back per workgroup): thread 0 only waits until its
  //    own counter operations are done before it counts itself out.
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    if (__hip_atomic_fetch_add(&counters[count], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P - 1) {
      for (int j = 0; j <= count; ++j) __hip_atomic_store(&counters[j], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

int chain_max_workgroups(int lds) {
  int dev = 0, cus = 0, per = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, tern_chain_kernel<2>, kChainThreads, (size_t)lds);
  if (e != hipSuccess) return -(int)e;
  return cus * per;
}

int device_cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return (int)e;
}

int copy_to_device(void* dst, const void* src, size_t bytes) {
  return (int)hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
}

int launch_chain(const ChainEntry* table, int count, int group, int workgroups, int lds, int* counters,
                 int* error_flag, int spin_limit, bool cooperative, void* stream) {
  if (count < 1 || workgroups < 1 || workgroups > kChainMaxWorkgroups || (group != 64 && group != 128))
    return (int)hipErrorInvalidValue;
  const int* wg_begin = (const int*)(table + count);
  const int2* work = (const int2*)(wg_begin + kChainMaxWorkgroups + 2);
  void* args[] = {(void*)&table, (void*)&count, (void*)&wg_begin, (void*)&work, (void*)&counters,
                  (void*)&error_flag, (void*)&spin_limit};
  const void* fn = group == 128 ? (const void*)tern_chain_kernel<2> : (const void*)tern_chain_kernel<4>;
  hipError_t e;
  if (cooperative) {
    // a workgroup that waits needs every other one resident: the launch
    // guarantees it or fails
    e = hipLaunchCooperativeKernel(fn, dim3(workgroups), dim3(kChainThreads), args, (unsigned)lds,
                                   (hipStream_t)stream);
  } else {
    // no waits: nothing depends on co-residency, an ordinary launch
    if (group == 128)
      hipLaunchKernelGGL(tern_chain_kernel<2>, dim3(workgroups), dim3(kChainThreads), (size_t)lds, (hipStream_t)stream,
                         table, count, wg_begin, work, counters, error_flag, spin_limit);
    else
      hipLaunchKernelGGL(tern_chain_kernel<4>, dim3(workgroups), dim3(kChainThreads), (size_t)lds, (hipStream_t)stream,
                         table, count, wg_begin, work, counters, error_flag, spin_limit);
    e = hipGetLastError();
  }
  return kernel_launched((int)e, TERN_KERNEL_CHAIN);
}

}  // namespace tern
