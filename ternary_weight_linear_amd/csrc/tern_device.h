// tern_device.h -- device-side helpers shared by the gfx950 kernels of this
// library.
// Internal, not installed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tern {
namespace dev {

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

// int8 B operand of v_mfma_i32_16x16x64_i8 from one packed code word (16
// weights): (word << 2i) & 0xC0C0C0C0 leaves every code in bits 7:6 of a byte,
// i.e. the int8 value 64*w (01 -> 64, 11 -> -64, 00 -> 0).
__device__ __forceinline__ i32x4 weights_operand_i8(uint32_t word) {
  return i32x4{(int)(word & 0xC0C0C0C0u), (int)((word << 2) & 0xC0C0C0C0u),
               (int)((word << 4) & 0xC0C0C0C0u), (int)((word << 6) & 0xC0C0C0C0u)};
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [p, p + bytes): loads past the end return zero,
// which is how absent tokens and rows read as zeros without branches.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // The descriptor lives in scalar registers: state that its inputs are
  // wave-uniform so the compiler never needs a per-lane loop to build it.
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           0x00020000);
}
constexpr int kAuxNontemporal = 2;  // "nt": streamed once, do not keep in cache
// A voffset past the end of every resource: the load is dropped and reads 0.
constexpr int kOffPastEnd = 0x40000000;

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

// ---- int8 limbs of bf16 activations (the gemv kernel, tern_limb.hip, and
// the small-T limb path, tern_limbtile.hip): per 256-wide k-tile, with
// 2^E <= max|x| < 2^(E+1) and d = E - 21, v = rne(x * 2^-d) is split into
// three balanced int8 digits v = l0 + 256 l1 + 65536 l2.

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Largest |x| over the 16 bf16 of a chunk (lo, hi), as a bf16 magnitude bit
// pattern (integer order = magnitude order), by packed 16-bit maxima.
__device__ __forceinline__ uint32_t absmax16(const u32x4& lo, const u32x4& hi) {
  u16x2 m = __builtin_bit_cast(u16x2, lo[0] & 0x7fff7fffu);
#pragma unroll
  for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, lo[i] & 0x7fff7fffu));
#pragma unroll
  for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, hi[i] & 0x7fff7fffu));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Max over the 16 lanes of a DPP row (each lane ends with the row's max).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  return v;
}

// Exponent shift of a k-tile from its largest magnitude m (a bf16 bit
// pattern): 2^E <= max|x| < 2^(E+1), d = E - 21.
__device__ __forceinline__ int limb_shift(uint32_t m) { return (int)(m >> 7) - 127 - 21; }

// Limb rows of one 16-element chunk. lo holds k = 2i, 2i+1 of the chunk's
// first 8 activations in dword i, hi the 8 activations 32 further on; dword i
// of limb row L gets the L-th digits of k = [32+2i, 2i, 33+2i, 2i+1] (the s8
// operand order).
//
// Per activation f = x * 2^-d + 1.5 * 2^23, one fma: the add rounds x * 2^-d
// to the nearest integer v (ties to even), so bits(f) = 0x4B400000 + v. The
// balanced base-256 digits v = l0 + 256 l1 + 65536 l2 are then byte 0 of
// bits(f), and, with w = bits(f) - 0x3F7F80 = 0x4B008080 + v, byte 1 of w
// with its top bit flipped and byte 2 of w (adding 0x80 below each digit
// makes the carries those of the balanced digits). Tiles whose maximum is
// below 2^-105 (d < -126, where 2^-d is no longer a float) scale x by 2^64
// first, which is exact.
template <bool TINY>
__device__ __forceinline__ void limb_chunk_t(const u32x4& lo, const u32x4& hi, float s, u32x4& o0, u32x4& o1,
                                             u32x4& o2) {
  constexpr float C = 12582912.0f;  // 1.5 * 2^23
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t e[4] = {lo[i] << 16, lo[i] & 0xffff0000u, hi[i] << 16, hi[i] & 0xffff0000u};  // xa xb ya yb
    uint32_t b[4], w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xj = TINY ? __uint_as_float(e[j]) * 0x1p64f : __uint_as_float(e[j]);
      b[j] = __float_as_uint(__builtin_fmaf(xj, s, C));
      w[j] = b[j] - 0x3F7F80u;
    }
    const uint32_t p0 = __builtin_amdgcn_perm(b[2], b[0], 0x0c0c0004u);    // [ya.0, xa.0, 0, 0]
    const uint32_t q0 = __builtin_amdgcn_perm(b[3], b[1], 0x0c0c0004u);    // [yb.0, xb.0, 0, 0]
    const uint32_t p12 = __builtin_amdgcn_perm(w[2], w[0], 0x02060105u);   // [ya.1, xa.1, ya.2, xa.2]
    const uint32_t q12 = __builtin_amdgcn_perm(w[3], w[1], 0x02060105u);   // [yb.1, xb.1, yb.2, xb.2]
    o0[i] = __builtin_amdgcn_perm(q0, p0, 0x05040100u);
    o1[i] = __builtin_amdgcn_perm(q12, p12, 0x05040100u) ^ 0x80808080u;
    o2[i] = __builtin_amdgcn_perm(q12, p12, 0x07060302u);
  }
}

__device__ __forceinline__ void limb_chunk(const u32x4& lo, const u32x4& hi, int d, u32x4& o0, u32x4& o1,
                                           u32x4& o2) {
  if (d < -126)
    limb_chunk_t<true>(lo, hi, __builtin_ldexpf(1.0f, -d - 64), o0, o1, o2);
  else
    limb_chunk_t<false>(lo, hi, __builtin_ldexpf(1.0f, -d), o0, o1, o2);
}
}  // namespace dev
}  // namespace tern
