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

// Largest |x| over 8 bf16 (as fp32 bit patterns: integer order = magnitude order).
__device__ __forceinline__ uint32_t absmax8(const u32x4& v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max((v[i] << 16) & 0x7fff0000u, v[i] & 0x7fff0000u));
  return m;
}

// Max over the 16 lanes of a DPP row (each lane ends with the row's max).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  return v;
}

// Fixed-point bits of one activation: f = x * 2^-d + 1.5 * 2^23 rounds x * 2^-d
// to the nearest integer v (ties to even) and holds 0x4B400000 + v. The limb
// bytes are then byte 0 of f, byte 1 of f + 128 and byte 2 of f + 32896 -
// 0x400000 (balanced base-256 digits of v; the 0x4B400000 offset does not
// reach bytes 0 and 1 and is taken out of byte 2).
struct LimbSrc {
  uint32_t u0, u1, u2;
};
__device__ __forceinline__ LimbSrc limb_src(uint32_t xbits_f32, int d) {
  const float f = __builtin_ldexpf(__uint_as_float(xbits_f32), -d) + 12582912.0f;
  const uint32_t b = __float_as_uint(f);
  return LimbSrc{b, b + 128u, b - 0x3F7F80u};
}

// Operand-order dword from four elements' limb sources: bytes [ya, xa, yb, xb]
// at byte position L of each (x = k 2i, 2i+1 of the low half, y = k 32+2i,
// 33+2i of the high half of the 64-wide block).
template <int L>
__device__ __forceinline__ uint32_t limb_dword(uint32_t xa, uint32_t xb, uint32_t ya, uint32_t yb) {
  constexpr uint32_t sel = (4u + L) | ((uint32_t)L << 8) | 0x0c0c0000u;
  const uint32_t p = __builtin_amdgcn_perm(ya, xa, sel);  // [ya.L, xa.L, 0, 0]
  const uint32_t q = __builtin_amdgcn_perm(yb, xb, sel);  // [yb.L, xb.L, 0, 0]
  return __builtin_amdgcn_perm(q, p, 0x05040100u);        // [ya.L, xa.L, yb.L, xb.L]
}
}  // namespace dev
}  // namespace tern
