// tern_chain.hip -- a whole decode pass (T = 1) over a chain of ternary
// projections in one launch, for the per-launch ramp and tail of short
// matrices: the pages replay each decode round as one captured graph of
// about 1224 kernels ("NINFER ternary perf-tuning" notes, section 6; "NInfer
// sm_89 fork" article, section 9 item 5), where every launch pays its own
// ramp and drain.
//
// One workgroup of 12 waves per CU. The host cuts the chain into stages at
// the items that depend on an item of the current stage, gives every
// workgroup one contiguous run of each stage's work (balanced by bytes of
// codes), and expands it into one record list per wave: its tasks (a strip
// and a range of k-tiles), and, the same in every wave of the workgroup and
// in the same order, the item switches, the signals after items that a later
// one waits on, and the ends of units. Work of an item with its K split over
// Wk waves (the gemv's plan) comes in units of 12 / Wk strips, each wave one
// K share of one strip, the shares added through LDS in ascending order;
// work of an item with Wk = 1 comes as single strips, dealt over the waves
// in turn.
//
// Streaming. Each wave walks its record list twice, once to request
// positions (strip, k-tile) and once to compute them, D positions apart: the
// codes and scales of its next D positions stay in flight in registers, so
// the weight stream does not stop at a unit's or an item's end. The
// positions are processed in groups of D with the ring slot of every
// position fixed at compile time, each slot reloaded right after its
// compute (the compiler's memory-counter waits then keep the whole ring in
// flight at every position); the records between positions (unit ends,
// item switches, waits, signals) are handled in each of the D steps.
//
// Limbs of x. The int8 limbs of the current item's activations live in one
// of two LDS slots; at an item switch the workgroup makes the next item's
// limbs in the other slot (every wave a share of the chunks, after its last
// position of the previous item) and passes one barrier, so waves still
// finishing the previous item keep reading theirs.
//
// Dependencies (after = j: items 0..j all finished) go through device-scope
// counters. Every value that crosses items (y, y_bf16, and x read from them)
// is stored and loaded with device-scope coherent accesses, the accesses of
// relaxed device-scope atomics, so no L2 write-back or invalidation is
// needed (each cost about 2-3 us per stage as fences): at a signal every
// wave waits for its stores to complete, the workgroup meets at a barrier
// and one thread adds one to the item's counter; at an item switch that
// needs it (the first of the workgroup's items with that dependency), thread
// 0 polls counter j until it reaches the number of workgroups (bounded by
// spin_limit, then it sets *error_flag and the workgroup skips the rest) and
// the workgroup meets at a barrier before it reads x. The last workgroup out
// zeroes the counters for the next launch.
//
// The arithmetic of a strip is the T = 1 integer-limb gemv of tern_limb.hip
// (limbs of x, codes decoded into i8 MFMA operands, per-group fp32 epilogue,
// k-tiles added in order, K shares added in ascending order), with the
// gemv's K split, so y is bit-identical to tern_linear's gemv rung.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

constexpr int kChainThreads = 64 * kChainWaves;
// Cache policy of the accesses that carry data between items: device
// (agent) scope, the encoding of a relaxed device-scope atomic access, which
// is coherent across the XCDs' L2 caches by itself (stores written through,
// loads not served from a stale line).
constexpr int kAuxAgent = 16;  // sc1
constexpr int kChainDepth = 8;  // positions of codes and scales in flight per wave

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);  // finite inputs
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS operations are
// complete, then s_barrier. Without the workgroup fence of __syncthreads(),
// which would also wait for the wave's outstanding global loads (the ring)
// and stores. The "memory" clobber keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  asm volatile("s_barrier" ::: "memory");
}

// Scalar loads of the chain table (read-only for the whole launch, written
// by the host before it). The compiler would read it with vector loads (it
// cannot tell that the kernel's stores leave it alone), and waiting for a
// vector load waits for every code load issued before it: the ring would
// drain at every unit. The wait is for the scalar counter only.
typedef int si4 __attribute__((ext_vector_type(4)));
typedef int si16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t a = (uint64_t)p;
  // readfirstlane returns an int: each half goes through uint32_t, or a low
  // word with bit 31 set would sign-extend into the high word
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ si4 sload4(const void* p) {
  si4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ si16 sload16(const void* p) {
  si16 v;
  asm volatile("s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_addr(p)) : "memory");
  return v;
}
// Fields of a ChainEntry from its first 64 bytes.
__device__ __forceinline__ const void* ent_ptr(const si16& v, int i) {
  return (const void*)(((uint64_t)(uint32_t)v[2 * i + 1] << 32) | (uint32_t)v[2 * i]);
}
constexpr int kEntCodes = 0, kEntScales = 1, kEntX = 2, kEntY = 3, kEntYb = 4;  // pointers
constexpr int kEntN = 10, kEntK = 11, kEntWn = 12, kEntWk = 13, kEntAfter = 15;  // ints
// Records of a wave's list: {type | item << 4, strip or unit, unit, kt0 | nkt << 16}.
constexpr int kRecTask = 0;      // a strip's k-tiles [kt0, kt0 + nkt), its sum to y (K not split)
constexpr int kRecTaskUnit = 1;  // one K share of a strip of unit `unit`, then the unit's reduction
constexpr int kRecUnit = 2;      // the reduction of unit `y` without a share of this wave
constexpr int kRecSwitch = 3;    // the workgroup moves to the item (y = 1: wait for its dependency; limbs)
constexpr int kRecSignal = 4;    // the workgroup is done with items 0..item
static_assert(offsetof(ChainEntry, n) == 4 * kEntN && offsetof(ChainEntry, after) == 4 * kEntAfter &&
                  offsetof(ChainEntry, y_bf16) == 8 * kEntYb && offsetof(ChainEntry, wk) == 4 * kEntWk,
              "ChainEntry field offsets");

// f(0) || f(1) || ... || f(D - 1) with compile-time indices, in order.
template <typename F, int... I>
__device__ __forceinline__ bool run_steps(F& f, std::integer_sequence<int, I...>) {
  return (f(std::integral_constant<int, I>{}) || ...);
}

template <int GPT>
__global__ void __launch_bounds__(kChainThreads) tern_chain_kernel(const int4* __restrict__ head, int count,
                                                                   int lds, int* __restrict__ counters,
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
  // The table's own layout against the launch: a table from another build
  // would put the limbs outside this launch's LDS.
  const int4 hd = head[0];
  const int rs = hd.x, slot_bytes = hd.y;
  if (hd.z != count || hd.w != (int)kChainTableMagic || rs < 64 || slot_bytes < 3 * rs ||
      2 * slot_bytes + 2 * kChainWaves * 16 * 4 > lds) {
    if (tid == 0) __hip_atomic_store(error_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const ChainEntry* __restrict__ table = (const ChainEntry*)(head + 1);
  // global, not flat, atomics: a pending flat operation makes every later
  // memory-counter wait a wait for zero
  __attribute__((address_space(1))) int* const gcount = (__attribute__((address_space(1))) int*)counters;
  __attribute__((address_space(1))) int* const gerror = (__attribute__((address_space(1))) int*)error_flag;
  const int* __restrict__ wv_begin = (const int*)(table + count);
  const si4* __restrict__ recs = (const si4*)(wv_begin + kChainRecordOffsets);
  if (tid == 0) s_abort = 0;
  __syncthreads();
  float* red = (float*)(smem + 2 * (size_t)slot_bytes);  // [2][12][16]: K-share sums of a unit
  const int wv = b * kChainWaves + wave;
  const int rec0 = wv_begin[wv], rec1 = wv_begin[wv + 1];

  // ---- load side: this wave's tasks in record order, D positions ahead
  int li = rec0;              // next record
  int litem = -1;             // item whose codes and scales lcodes, lscales point to
  const void* lcodes = nullptr;
  const void* lscales = nullptr;
  int lKT = 0;                // k-tiles of litem
  int lkt0 = 0, lnkt = 0, lj = 0;  // current task: k-tiles [lkt0, lkt0 + lnkt), next lj
  bool lend = false;          // past the last task
  rsrc_t lcr = make_rsrc(table, 0), lsr = lcr;  // codes and scales of the task (none yet: loads read zeros)
  auto lnext_task = [&]() {   // to the next task record (or to the end)
    for (;;) {
      if (li >= rec1) {       // the end: stay on the last task's last position
        lend = true;
        lj = max(lnkt - 1, 0);
        return;
      }
      const si4 e = sload4(recs + li++);
      const int type = e.x & 15;
      if (type > kRecTaskUnit) continue;  // no positions
      const int item = e.x >> 4;
      if (item != litem) {
        const si16 c = sload16(table + item);
        lcodes = ent_ptr(c, kEntCodes);
        lscales = ent_ptr(c, kEntScales);
        lKT = c[kEntK] >> 8;
        litem = item;
      }
      lkt0 = e.w & 0xffff;
      lnkt = e.w >> 16;
      lcr = make_rsrc((const char*)lcodes + (size_t)e.y * lKT * 1024, (uint32_t)lKT * 1024);
      lsr = make_rsrc((const char*)lscales + (size_t)e.y * lKT * 32 * GPT, (uint32_t)lKT * 32 * GPT);
      lj = 0;
      return;
    }
  };
  struct Slot {
    u32x4 P;
    uint32_t sw[GPT / 2];
  };
  // The next position into s, then one on. Past the last task the last
  // position is read again (a wave without tasks reads zeros: its resource
  // holds no bytes), so that every load is issued the same way and the
  // ring's memory-counter waits stay exact.
  auto lload = [&](Slot& s) {
    const int kt = __builtin_amdgcn_readfirstlane(lkt0 + lj);
    s.P = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(lcr, lane * 16, kt * 1024, kAuxNontemporal));
    if (GPT == 2) {
      s.sw[0] = __builtin_amdgcn_raw_buffer_load_b32(lsr, r * GPT * 2, kt * 32 * GPT, 0);
    } else {
      const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(lsr, r * GPT * 2, kt * 32 * GPT, 0);
      s.sw[0] = w2[0];
      s.sw[GPT / 2 - 1] = w2[1];
    }
    if (!lend && ++lj == lnkt) lnext_task();
  };

  // ---- compute side: every record of this wave, in order
  int ci = rec0;             // next record
  int ckt0 = 0, cnkt = 0, cj = 0;  // current task
  int cstrip = 0, cunit = 0, ctype = 0;
  bool cend = false;
  int lslot = 1;             // LDS slot of the limbs in use (the first item takes slot 0)
  int units_done = 0;        // Wk > 1 units passed (parity of red)
  int cwn = 1, cwk = 1, cNS = 0;  // plan of the current item
  float total = 0.f;
  rsrc_t ys = make_rsrc(table, 0), ybs = ys;  // y and y_bf16 of the current item (0 bytes: no y_bf16)
  const char* abase = nullptr;
  const int* dexp = nullptr;

  // Limbs of item i into the other LDS slot, after its wait (the whole
  // workgroup passes here together).
  auto item_switch = [&](const si16& e, bool wait) {
    const int after = e[kEntAfter];
    if (wait && after >= 0) {
      if (tid == 0) {
        bool ok = false;
        for (int it = 0;; ++it) {
          if (__hip_atomic_load(&gcount[after], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= P) {
            ok = true;
            break;
          }
          if (__hip_atomic_load(gerror, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
          if (it >= spin_limit) {
            __hip_atomic_store(gerror, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (!ok) s_abort = 1;
      }
      lds_barrier();
      if (s_abort) return;
    }
    lslot ^= 1;
    char* base = smem + (size_t)lslot * slot_bytes;
    int* dx = (int*)(base + 3 * (size_t)rs);
    const int K = e[kEntK];
    const rsrc_t xr = make_rsrc(ent_ptr(e, kEntX), (uint32_t)K * 2);
    for (int c = tid; c < (K >> 4); c += kChainThreads) {  // rows of 16 lanes are wholly in or out
      const int off = 64 * (c >> 2) + 8 * (c & 3);
      const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, off * 2, 0, kAuxAgent));
      const u32x4 hi =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (off + 32) * 2, 0, kAuxAgent));
      const int d = limb_shift(row16_max_u32(absmax16(lo, hi)));
      u32x4 o0, o1, o2;
      limb_chunk(lo, hi, d, o0, o1, o2);
      char* row = base + 16 * c;
      *(u32x4*)row = o0;
      *(u32x4*)(row + rs) = o1;
      *(u32x4*)(row + 2 * rs) = o2;
      if ((c & 15) == 0) dx[c >> 4] = d;
    }
    lds_barrier();
    // the item's plan and outputs
    cwn = e[kEntWn];
    cwk = e[kEntWk];
    cNS = e[kEntN] >> 4;
    const void* yb = ent_ptr(e, kEntYb);
    ys = make_rsrc(ent_ptr(e, kEntY), (uint32_t)e[kEntN] * 4);
    ybs = make_rsrc(yb, yb ? (uint32_t)e[kEntN] * 2 : 0u);
    abase = base + (size_t)(r < 3 ? r : 0) * rs + 16 * g;
    dexp = (const int*)(base + 3 * (size_t)rs);
  };
  // A signal: this workgroup is done with items 0..i. Its outputs went out
  // as device-coherent stores, so once they have completed (the wait, every
  // wave, then the barrier) they are visible to every XCD, and no L2
  // write-back is needed before the count.
  auto signal = [&](int i) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    lds_barrier();                  // ... and every other wave's
    if (tid == 0) __hip_atomic_fetch_add(&gcount[i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // Output o of the current item: device-coherent buffer stores (written
  // through to where every XCD reads them; a flat store would also make the
  // compiler wait for every outstanding load before the next position).
  auto store_y = [&](size_t o, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ys, (int)o * 4, 0, kAuxAgent);
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), ybs, (int)o * 2, 0, kAuxAgent);  // dropped without y_bf16
  };
  // End of unit u of a Wk > 1 item (with this wave's share, or without):
  // the shares meet in LDS, the first threads add them in ascending order
  // and store.
  auto unit_end = [&](int u, bool share) {
    float* rb = red + (units_done & 1) * (kChainWaves * 16);
    const int wn = wave % cwn, wk = wave / cwn;
    if (share && lane < 16) rb[(wk * cwn + wn) * 16 + lane] = total;
    lds_barrier();
    const int nsb = min(cwn, cNS - u * cwn);
    if (tid < nsb * 16) {
      const int ls = tid >> 4, col = tid & 15;
      float sum = 0.f;
      for (int w = 0; w < cwk; ++w) sum += rb[(w * cwn + ls) * 16 + col];
      store_y((size_t)(u * cwn + ls) * 16 + col, sum);
    }
    ++units_done;
  };
  // To the next task record, doing the work of the records between
  // (item switches, waits, signals, unit ends without a share).
  auto cnext_task = [&]() {
    for (;;) {
      if (ci >= rec1) {
        cend = true;
        return;
      }
      const si4 e = sload4(recs + ci++);
      const int type = e.x & 15;
      if (type == kRecSwitch) {
        item_switch(sload16(table + (e.x >> 4)), e.y != 0);
        if (s_abort) {
          cend = true;
          return;
        }
      } else if (type == kRecSignal) {
        signal(e.x >> 4);
      } else if (type == kRecUnit) {
        unit_end(e.y, false);
      } else {
        ctype = type;
        cstrip = e.y;
        cunit = e.z;
        ckt0 = e.w & 0xffff;
        cnkt = e.w >> 16;
        total = 0.f;
        cj = 0;
        return;
      }
    }
  };
  // End of the current task: its sum to y, or to its unit's reduction.
  auto task_end = [&]() {
    if (ctype == kRecTask) {
      if (lane < 16) store_y((size_t)cstrip * 16 + lane, total);
    } else {
      unit_end(cunit, true);
    }
  };
  // One position: the k-tile cj of the current task from ring slot s.
  auto compute = [&](const Slot& s) {
    const int kt = ckt0 + cj;
    i32x4 a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = *(const i32x4*)(abase + 64 * (4 * kt + q));
    const int dsh = dexp[kt] - 6;
    float part = 0.f;
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      i32x4 acc = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KBPG; ++kk) {
        const int q = gi * KBPG + kk;
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[q], weights_operand_i8(s.P[q]), acc, 0, 0, 0);
      }
      const uint32_t spair = s.sw[gi >> 1];
      const float sc = half_bits_to_float((uint16_t)((gi & 1) ? (spair >> 16) : (spair & 0xffffu)));
      const int low = (int)(((uint32_t)acc[1] << 8) + (uint32_t)acc[0]);  // 256 a1 + a0
      const float v = __builtin_fmaf(65536.0f, (float)acc[2], (float)low);
      part = gi == 0 ? sc * v : __builtin_fmaf(sc, v, part);
    }
    total += __builtin_ldexpf(part, dsh);
  };

  // ---- the stream. The first D positions are requested before the first
  // item's limbs are made.
  lnext_task();
  {
    Slot ring[D];
#pragma unroll
    for (int j = 0; j < D; ++j) lload(ring[j]);
    cnext_task();
    if (cend) goto stream_done;
    // One position: compute slot S (a compile-time constant), then request
    // the position D ahead into it. True at the end of the stream. (Each
    // slot is reloaded right after its own compute, so every wait finds the
    // same D positions in flight.)
    auto step = [&](auto slot) {
      constexpr int S = decltype(slot)::value;
      compute(ring[S]);
      __builtin_amdgcn_sched_barrier(0);
      lload(ring[S]);
      if (++cj == cnkt) {
        task_end();
        cnext_task();
      }
      return cend;
    };
    while (!run_steps(step, std::make_integer_sequence<int, D>{})) {
    }
  }
stream_done:

  // The last workgroup out zeroes the counters for the next launch. No data
  // is published here (the kernel's end does that), so no release fence:
  // thread 0 only waits until its own counter operations are done.
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    if (__hip_atomic_fetch_add(&gcount[count], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P - 1) {
      for (int j = 0; j <= count; ++j) __hip_atomic_store(&gcount[j], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

int launch_chain(const void* table, int count, int group, int workgroups, int lds, int* counters, int* error_flag,
                 int spin_limit, bool cooperative, void* stream) {
  if (count < 1 || workgroups < 1 || workgroups > kChainMaxWorkgroups || (group != 64 && group != 128))
    return (int)hipErrorInvalidValue;
  const int4* head = (const int4*)table;
  void* args[] = {(void*)&head, (void*)&count, (void*)&lds, (void*)&counters, (void*)&error_flag,
                  (void*)&spin_limit};
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
                         head, count, lds, counters, error_flag, spin_limit);
    else
      hipLaunchKernelGGL(tern_chain_kernel<4>, dim3(workgroups), dim3(kChainThreads), (size_t)lds, (hipStream_t)stream,
                         head, count, lds, counters, error_flag, spin_limit);
    e = hipGetLastError();
  }
  return kernel_launched((int)e, TERN_KERNEL_CHAIN);
}

}  // namespace tern
