// tern_probe.hip -- streaming-read ceiling of the part, for reporting the
// layer kernels' bandwidth against what one launch can read at all.
//
// The tuning notes on the pages measure a read-only bandwidth ceiling on
// their card next to the kernels ("NINFER ternary perf-tuning" notes,
// section 6, the table of measured constants) and rate the decode kernels
// against it. This kernel is that measurement on gfx950: it reads a buffer
// once with 128-bit non-temporal loads and does no other work, so the time
// of one launch over B bytes is the floor of any single-launch kernel that
// must stream B bytes (launch, ramp and drain included).
//
// Each wave reads its own contiguous run of `per_wave` KiB, 1 KiB (64 lanes
// x 16 B) per load instruction, keeping D loads in flight in a register
// ring. The loads are XOR-folded into one word per lane, which is stored
// only if it equals an arbitrary constant, so the loads cannot be dropped
// and in practice nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

template <int D>
__global__ void __launch_bounds__(256) tern_stream_read_kernel(const char* __restrict__ buf, uint32_t kib,
                                                               uint32_t per_wave, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * 4u + (threadIdx.x >> 6);
  const uint32_t first = wave * per_wave;
  if (first >= kib) return;
  const uint32_t n = min(per_wave, kib - first);
  // The resource covers this wave's run only: loads past it return zero.
  const rsrc_t rs = make_rsrc(buf + (size_t)first * 1024, n * 1024u);
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j)
    ring[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + j * 1024, 0,
                                                                              kAuxNontemporal));
  for (uint32_t i = 0; i < n; i += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      acc ^= ring[j];
      const uint32_t next = i + j + D;
      const int off = next < n ? (int)(next * 1024u) + lane * 16 : kOffPastEnd;
      ring[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kAuxNontemporal));
    }
  }
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9E3779B9u) sink[0] = r;
}

template <int D>
void launch_d(const void* buf, uint32_t kib, uint32_t per_wave, uint32_t waves, uint32_t* sink, hipStream_t st) {
  const dim3 grid((waves + 3) / 4);
  hipLaunchKernelGGL((tern_stream_read_kernel<D>), grid, dim3(256), 0, st, (const char*)buf, kib, per_wave, sink);
}

}  // namespace

int launch_stream_read(const void* buf, size_t bytes, int depth, int waves_per_cu, uint32_t* sink, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const uint32_t kib = (uint32_t)(bytes / 1024);
  // Spread the runs over waves_per_cu waves on each of the 256 CUs.
  const uint32_t target = 256u * (uint32_t)waves_per_cu;
  const uint32_t per_wave = (kib + target - 1) / target;
  const uint32_t waves = (kib + per_wave - 1) / per_wave;
  switch (depth) {
    case 4: launch_d<4>(buf, kib, per_wave, waves, sink, st); break;
    case 8: launch_d<8>(buf, kib, per_wave, waves, sink, st); break;
    case 16: launch_d<16>(buf, kib, per_wave, waves, sink, st); break;
    default: return (int)hipErrorInvalidValue;
  }
  return kernel_launched((int)hipGetLastError(), TERN_KERNEL_STREAM_READ);
}

}  // namespace tern
