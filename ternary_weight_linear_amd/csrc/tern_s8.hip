// tern_s8.hip -- gfx950 kernels of the s8 rung: per-token int8 activation
// quantisation and the int8 x ternary contraction on the i8 matrix cores.
// Built with the MFMA results kept in VGPRs (the fp32 scale epilogue reads
// every accumulator), see build.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tern_device.h"
#include "tern_internal.h"

namespace tern {
namespace {
using namespace dev;

// --------------------------------------------------------------------------
// per-token int8 activation quantisation
// --------------------------------------------------------------------------

__device__ __forceinline__ uint32_t quant_code(float v, float sc) {
  const float r = rintf(v / sc);  // IEEE division, ties-to-even rounding
  const float c = fminf(fmaxf(r, -127.f), 127.f);
  return (uint32_t)((int)c) & 0xffu;
}
__device__ __forceinline__ uint32_t quant_byte(uint32_t xbits, float sc) {
  return quant_code(__uint_as_float(xbits), sc);
}

// The same code from y = fl(v * r), r = fl(1 / sc), sc a normal float: with
// |v| <= 127 sc, y is within 2^-16 of v / sc and the IEEE quotient within
// 2^-17, so unless y lies within 2^-15 of a half-integer both round to the
// same integer. Such values set `near`, and the caller redoes them with the
// division.
__device__ __forceinline__ uint32_t quant_code_rcp(float v, float r, bool& near) {
#pragma clang fp contract(off)
  const float y = v * r;
  const float t = rintf(y);
  near |= !(fabsf(y - t) < 0.5f - 0x1p-15f);
  const float c = fminf(fmaxf(t, -127.f), 127.f);
  return (uint32_t)((int)c) & 0xffu;
}

// Codes of 16 values (4 dwords, byte e of dword d = value 4d + e): by the
// reciprocal when the token's scale allows it and no value is near a rounding
// boundary, else by division.
__device__ __forceinline__ void quant_codes16(const float (&v)[16], float sc, float r, bool rcp_ok,
                                              uint32_t (&w)[4]) {
  bool near = !rcp_ok;
  if (rcp_ok) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
      w[d] = quant_code_rcp(v[4 * d], r, near) | (quant_code_rcp(v[4 * d + 1], r, near) << 8) |
             (quant_code_rcp(v[4 * d + 2], r, near) << 16) | (quant_code_rcp(v[4 * d + 3], r, near) << 24);
  }
  if (near) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
      w[d] = quant_code(v[4 * d], sc) | (quant_code(v[4 * d + 1], sc) << 8) |
             (quant_code(v[4 * d + 2], sc) << 16) | (quant_code(v[4 * d + 3], sc) << 24);
  }
}

// The s8 kernel's operand order inside every 64-byte k-block kb: byte
// 16g + 4i + beta holds k = 64kb + 8g + kmap(i, beta) with
// kmap(i, .) = {32 + 2i, 2i, 33 + 2i, 2i + 1}. It is the order in which
// (word << 2i) & 0xC0C0C0C0 lays out the codes of a packed weight word (see
// weights_operand_i8), so activations stored this way feed the MFMA as is.
// From the natural order (lo = bytes 8g..8g+7, hi = bytes 32+8g..32+8g+7 of
// the block) each dword is one byte permute.
__device__ __forceinline__ u32x4 s8_operand_order(uint32_t L0, uint32_t L1, uint32_t H0,
                                                  uint32_t H1) {
  return u32x4{__builtin_amdgcn_perm(H0, L0, 0x01050004u), __builtin_amdgcn_perm(H0, L0, 0x03070206u),
               __builtin_amdgcn_perm(H1, L1, 0x01050004u), __builtin_amdgcn_perm(H1, L1, 0x03070206u)};
}

// Per-token quantisation. One block per token: absmax (DPP wave reduction,
// then across the 4 waves), scale = absmax / 127, then the codes. PERM writes
// them in the s8 operand order (K % 64 == 0), otherwise row-major.
template <bool PERM>
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
  auto codes8 = [&](const uint4 v, uint32_t& lo, uint32_t& hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b[2 * i] = quant_byte(w[i] << 16, sc);
      b[2 * i + 1] = quant_byte(w[i] & 0xffff0000u, sc);
    }
    lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
  };
  if (!PERM) {
    uint2* qr = (uint2*)(q + (size_t)t * K);
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      uint2 out = uint2{0u, 0u};
      if (am != 0) codes8(xr[c], out.x, out.y);
      qr[c] = out;
    }
  } else {
    // output chunk j (16 bytes) = group g = j & 3 of 64-byte block j >> 2
    u32x4* qr = (u32x4*)(q + (size_t)t * K);
    for (int j = threadIdx.x; j < (K >> 4); j += 256) {
      u32x4 out = u32x4{0u, 0u, 0u, 0u};
      if (am != 0) {
        const int blk = j >> 2, g = j & 3;
        uint32_t L0, L1, H0, H1;
        codes8(xr[blk * 8 + g], L0, L1);      // k = 64 blk + 8g .. +7
        codes8(xr[blk * 8 + 4 + g], H0, H1);  // k = 64 blk + 32 + 8g .. +7
        out = s8_operand_order(L0, L1, H0, H1);
      }
      qr[j] = out;
    }
  }
}

// Single-pass variant of the operand-order quantisation for K <= NT * 16 * NU:
// thread i holds the activations of output chunks i, i + NT, ... in
// registers (both 8-element halves of each), so x is read once and all of
// its loads go out before the absmax reduction. NT = 256 threads per token
// for long batches; 1024 for short ones, where the few workgroups are a
// latency chain and four times the threads make it a quarter as long.
template <int NU, int NT>
__global__ void __launch_bounds__(NT) tern_quant_s8_perm_kernel(const uint16_t* __restrict__ x, int K,
                                                                int8_t* __restrict__ q,
                                                                float* __restrict__ scale) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t wmax[NW];
  const int t = blockIdx.x;
  const uint4* xr = (const uint4*)(x + (size_t)t * K);
  const int nu = K >> 4;  // 16-byte output chunks of the token
  uint4 lo[NU], hi[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int j = threadIdx.x + NT * u;
    if (j < nu) {
      const int blk = j >> 2, g = j & 3;
      lo[u] = xr[blk * 8 + g];      // k = 64 blk + 8g .. +7
      hi[u] = xr[blk * 8 + 4 + g];  // k = 64 blk + 32 + 8g .. +7
    } else {
      lo[u] = hi[u] = uint4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t m16 = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u)
    m16 = max(m16, absmax16(u32x4{lo[u].x, lo[u].y, lo[u].z, lo[u].w}, u32x4{hi[u].x, hi[u].y, hi[u].z, hi[u].w}));
  uint32_t m = wave_max_u32(m16 << 16);  // as an fp32 bit pattern
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t am = wmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) am = max(am, wmax[w]);
  const float sc = __uint_as_float(am) / 127.0f;  // IEEE single division
  if (threadIdx.x == 0) scale[t] = am == 0 ? 0.0f : sc;
  // Codes by the reciprocal (quant_code_rcp); the 8 values of a 16-byte load
  // are redone by division when one of them lies near a rounding boundary,
  // from the same packed registers, so no more values stay live.
  const float r = 1.0f / sc;
  const bool rcp_ok = sc >= 0x1p-126f;  // a normal scale: r is finite
  u32x4* qr = (u32x4*)(q + (size_t)t * K);
  auto codes8 = [&](const uint4 v, uint32_t& c0, uint32_t& c1) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t b[8];
    bool near = !rcp_ok;
    if (rcp_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[2 * i] = quant_code_rcp(__uint_as_float(w[i] << 16), r, near);
        b[2 * i + 1] = quant_code_rcp(__uint_as_float(w[i] & 0xffff0000u), r, near);
      }
    }
    if (near) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[2 * i] = quant_byte(w[i] << 16, sc);
        b[2 * i + 1] = quant_byte(w[i] & 0xffff0000u, sc);
      }
    }
    c0 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    c1 = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
  };
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int j = threadIdx.x + NT * u;
    if (j >= nu) break;
    u32x4 out = u32x4{0u, 0u, 0u, 0u};
    if (am != 0) {
      // An empty asm that takes the chunk's packed words as read and
      // rewritten here keeps the compiler from unpacking every chunk to fp32
      // right after the loads (twice the registers: 102 instead of 63 VGPRs
      // at NU = 5); no instruction is emitted.
      asm volatile("" : "+v"(lo[u].x), "+v"(lo[u].y), "+v"(lo[u].z), "+v"(lo[u].w), "+v"(hi[u].x), "+v"(hi[u].y),
                   "+v"(hi[u].z), "+v"(hi[u].w));
      uint32_t L0, L1, H0, H1;
      codes8(lo[u], L0, L1);
      codes8(hi[u], H0, H1);
      out = s8_operand_order(L0, L1, H0, H1);
    }
    qr[j] = out;
  }
}

// --------------------------------------------------------------------------
// rotated per-token int8 quantisation
// --------------------------------------------------------------------------
//
// xr = (1/32) H x on every 1024-wide block of a token (H the Sylvester
// Hadamard matrix of order 1024), then the quantisation above applied to xr.
// The pages fold the rotation of the original ternary model into the
// activation quantisation ("NInfer sm_89 fork" article, section 9 item 2) and
// rotate 1024-wide blocks ("NINFER ternary perf-tuning" notes, section 6,
// constants table); their rotation kernel, one warp per (block, token), was
// bound by launch latency, not by its traffic.
//
// The rotation is computed in fp32 as the fast Walsh-Hadamard transform with
// strides 1, 2, ..., 512 in that order, each pair (i, i + h) becoming
// (u + v, u - v) with one rounding each, then a multiply by 1/32: fixing the
// order fixes every rounding, so the codes are reproducible bit for bit.
//
// One workgroup per token; wave w rotates blocks w, w + 4, ... and keeps the
// results in registers (NBW blocks at most) until the token's absmax is
// known. Per block a lane holds 16 values in three layouts, element index i
// (10 bits) split between 4 register bits and 6 lane bits:
//   P1  i = 16 l + j                         (registers: bits 0-3)
//   P2  i = (l & 15) + 16 j + 256 (l >> 4)  (registers: bits 4-7)
//   P3  registers j: bits 0-2 and 5; lane l: bits 3-4, 6-7, 8-9 (l >> 4)
// Strides 1..8 and 16..128 run inside the registers of P1 and P2; strides 256
// and 512 pair lanes l and l ^ 16, l ^ 32 of P3, where the lane holding u
// computes fma(+1, u, v) = u + v and the one holding v fma(-1, v, u) = u - v.
// P3 is the output layout: a lane's 16 values are the k = 8g..8g+7 and
// 32+8g..32+8g+7 of one 64-wide k-block, i.e. one 16-byte chunk of the s8
// operand order (or two 8-byte pieces of a row-major row). The relayouts go
// through 4 KiB of LDS per wave, positions XOR-swizzled so that all three
// layouts read and write without bank conflicts.
constexpr int kRotBlock = 1024;

__device__ __forceinline__ int rot_pos(int i) {
  return i ^ (((i >> 5) & 1) << 3) ^ (((i >> 6) & 3) << 1) ^ (((i >> 8) & 1) * 17);
}
__device__ __forceinline__ int rot_p2(int l, int j) { return (l & 15) + 16 * j + 256 * (l >> 4); }
__device__ __forceinline__ int rot_p3(int l, int j) {
  return (j & 7) | ((l & 3) << 3) | ((j >> 3) << 5) | (((l >> 2) & 3) << 6) | ((l >> 4) << 8);
}

// All lanes' LDS accesses before this point are ordered before those after it
// (LDS instructions of a wave execute in order; this keeps the compiler from
// moving them across).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The strides whose element bit lives in register bit 0..3.
__device__ __forceinline__ void fwht_regs16(float (&z)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (!(j & h)) {
        const float u = z[j], v = z[j + h];
        z[j] = u + v;
        z[j + h] = u - v;
      }
}

template <int NBW, bool PERM>
__global__ void __launch_bounds__(256) tern_quant_rot_kernel(const uint16_t* __restrict__ x, int K,
                                                             int8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
  __shared__ float xbuf[4][kRotBlock];
  __shared__ uint32_t wmax[4];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = K >> 10;
  float* sb = xbuf[wave];
  const float sg16 = (lane & 16) ? -1.0f : 1.0f;
  const float sg32 = (lane & 32) ? -1.0f : 1.0f;

  float v[NBW][16];
  uint32_t m = 0;
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
    const int b = wave + 4 * jb;
    if (b >= nb) break;  // wave-uniform
    float z[16];
    {  // P1: 16 consecutive activations per lane
      const uint16_t* src = x + (size_t)t * K + (size_t)b * kRotBlock + 16 * lane;
      const u32x4 lo = *(const u32x4*)src;
      const u32x4 hi = *(const u32x4*)(src + 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[2 * i] = __uint_as_float(lo[i] << 16);
        z[2 * i + 1] = __uint_as_float(lo[i] & 0xffff0000u);
        z[8 + 2 * i] = __uint_as_float(hi[i] << 16);
        z[9 + 2 * i] = __uint_as_float(hi[i] & 0xffff0000u);
      }
    }
    fwht_regs16(z);  // strides 1, 2, 4, 8
#pragma unroll
    for (int j = 0; j < 16; ++j) sb[rot_pos(16 * lane + j)] = z[j];
    wave_lds_order();
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = sb[rot_pos(rot_p2(lane, j))];
    wave_lds_order();
    fwht_regs16(z);  // strides 16, 32, 64, 128
#pragma unroll
    for (int j = 0; j < 16; ++j) sb[rot_pos(rot_p2(lane, j))] = z[j];
    wave_lds_order();
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = sb[rot_pos(rot_p3(lane, j))];
    wave_lds_order();
    // stride 256: lanes l, l ^ 16 (ds_swizzle, xor mask 16 within 32 lanes)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(z[j]), 0x401f));
      z[j] = __builtin_fmaf(sg16, z[j], p);
    }
    // stride 512: lanes l, l ^ 32
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(z[j])));
      z[j] = __builtin_fmaf(sg32, z[j], p);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      v[jb][j] = z[j] * 0.03125f;
      m = max(m, __float_as_uint(v[jb][j]) & 0x7fffffffu);
    }
  }
  m = wave_max_u32(m);
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  const uint32_t am = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float sc = __uint_as_float(am) / 127.0f;  // IEEE single division
  if (threadIdx.x == 0) scale[t] = am == 0 ? 0.0f : sc;
  const float r = 1.0f / sc;
  const bool rcp_ok = sc >= 0x1p-126f;  // a normal scale: r is finite

  // P3 lane l: 64-wide k-block c = ((l >> 2) & 3) + 4 (l >> 4) of the 1024
  // block, 8-wide group g = l & 3; register j = (k & 7) + 8 * (k >= 32).
  const int g = lane & 3, c = ((lane >> 2) & 3) | ((lane >> 4) << 2);
#pragma unroll
  for (int jb = 0; jb < NBW; ++jb) {
    const int b = wave + 4 * jb;
    if (b >= nb) break;
    uint32_t w4[4] = {0u, 0u, 0u, 0u};  // codes of k = 8g+0..3, 8g+4..7, 32+8g+0..3, 32+8g+4..7
    if (am != 0) quant_codes16(v[jb], sc, r, rcp_ok, w4);
    int8_t* dst = q + (size_t)t * K + (size_t)b * kRotBlock + 64 * c;
    if (PERM) {
      *(u32x4*)(dst + 16 * g) = s8_operand_order(w4[0], w4[1], w4[2], w4[3]);
    } else {
      *(uint2*)(dst + 8 * g) = uint2{w4[0], w4[1]};
      *(uint2*)(dst + 32 + 8 * g) = uint2{w4[2], w4[3]};
    }
  }
}

// --------------------------------------------------------------------------
// s8 kernel: int8 activations x ternary weights on the i8 matrix cores
// --------------------------------------------------------------------------
//
// Block: 4 waves, tile of 64 tokens x 256 outputs; wave w owns the 64 x 64
// block of outputs [64w, 64w + 64) = 4 strips, as 4 x 4 v_mfma_i32_16x16x64_i8
// tiles (A = activations, rows = tokens; B = weights, columns = outputs).
// Per 256-wide k-tile:
//  * the block's 64 x 256 activation tile goes to LDS (double buffered) by
//    direct buffer-to-LDS loads, rows of 256 bytes with the 16-byte chunks of
//    row r stored at chunk index (c ^ (r & 15)) so that the 16 rows of an
//    operand fragment read without bank conflicts; the 4 waves share it;
//  * each wave reads its own 4 strips' packed codes with one 16-byte load per
//    lane per strip -- exactly the lane's B-operand codes -- and decodes each
//    word into an MFMA operand with one shift and one mask per 4 weights:
//    (word << 2i) & 0xC0C0C0C0 leaves every code in bits 7:6 of a byte, i.e.
//    the int8 value 64*w. The MFMA accumulates 64*acc (|64*acc| <= 64*127*G,
//    exact in int32 and in fp32), and the 2^-6 goes into the fp32 scale:
//    fma(float(64*acc), s/64, total) rounds exactly like fma(acc, s, total);
//  * epilogue per scale group and strip: total = fma(float(acc), s[n][g],
//    total), groups ascending; at the end y = total * scale_t.

constexpr int kS8BM = 64;


template <int GPT>
struct S8Stage {
  u32x4 code[4];            // the lane's 16 bytes of each of the wave's 4 strips
  uint32_t sw[4][GPT / 2];  // fp16 scale pairs of row (lane & 15) of each strip
};

template <int GPT, bool DEBUG_ACC, bool QPERM>
__global__ void __launch_bounds__(256) tern_s8_kernel(const int8_t* __restrict__ q,
                                                      const float* __restrict__ act_scale, int T,
                                                      int K, const u32x4* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      float* __restrict__ y,
                                                      int32_t* __restrict__ acc_out, int N) {
  __shared__ __attribute__((aligned(1024))) int8_t As[2][kS8BM * 256];
  __shared__ float sas[kS8BM];
  constexpr int KBPG = 4 / GPT;  // 64-wide k-blocks per scale group
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;
  const int NS = N >> 4;
  const int KT = K >> 8;
  const int NG = K / (256 / GPT);
  const int t0 = blockIdx.y * kS8BM;
  const int nt = min(kS8BM, T - t0);
  const int st0 = blockIdx.x * 16 + wave * 4;  // first strip of this wave
  const int nst = max(0, min(4, NS - st0));     // strips of this wave that exist

  const rsrc_t qr = make_rsrc(q + (size_t)t0 * K, (uint32_t)nt * K);
  const rsrc_t cr = make_rsrc(codes + (size_t)min(st0, NS) * KT * 64, (uint32_t)nst * KT * 1024);
  const rsrc_t sr = make_rsrc(scales + (size_t)min(st0, NS) * KT * 16 * GPT,
                              (uint32_t)nst * KT * 16 * GPT * 2);

  // Activation staging. QPERM (q already in operand order): wave w loads rows
  // 16w .. 16w+15 with 4 direct-to-LDS loads of 4 rows each; lane i of load j
  // writes LDS chunk (row 16w + 4j + i/16, chunk i % 16) and so fetches the
  // global chunk (i % 16) ^ (row & 15). Otherwise (row-major q): thread ->
  // (row, 64-byte block), byte permute in registers, then ds_write.
  const int qrow_d = 16 * wave + (lane >> 4);  // + 4j
  auto stage_a_direct = [&](int kt, int buf) {
    kt = __builtin_amdgcn_readfirstlane(kt);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = qrow_d + 4 * j;
      const int chunk = (lane & 15) ^ (row & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qr, (__attribute__((address_space(3))) void*)&As[buf][(16 * wave + 4 * j) * 256], 16,
          row * K + chunk * 16, kt * 256, 0, kAuxNontemporal);
    }
  };
  const int arow = tid >> 2, ablk = tid & 3;
  auto load_a_regs = [&](int kt, u32x4 (&v)[4]) {
    kt = __builtin_amdgcn_readfirstlane(kt);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      v[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           qr, arow * K + ablk * 64 + 16 * c, kt * 256, 0));
  };
  auto store_a_regs = [&](int buf, const u32x4 (&v)[4]) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const u32x4 lo = v[gg >> 1], hi = v[2 + (gg >> 1)];
      const int d = (gg & 1) * 2;
      const int chunk = (ablk * 4 + gg) ^ (arow & 15);
      *(u32x4*)&As[buf][arow * 256 + chunk * 16] =
          s8_operand_order(lo[d], lo[d + 1], hi[d], hi[d + 1]);
    }
  };
  auto load_w = [&](int kt, S8Stage<GPT>& b) {
    kt = __builtin_amdgcn_readfirstlane(kt);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int je = min(j, max(nst - 1, 0));
      b.code[j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, lane * 16, (je * KT + kt) * 1024,
                                                       kAuxNontemporal));
      const int soff = (je * KT + kt) * 16 * GPT * 2;
      if (GPT == 2) {
        b.sw[j][0] = __builtin_amdgcn_raw_buffer_load_b32(sr, r * GPT * 2, soff, 0);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(sr, r * GPT * 2, soff, 0);
        b.sw[j][0] = v[0];
        b.sw[j][GPT / 2 - 1] = v[1];
      }
    }
  };

  f32x4 tot[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) tot[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kt, int buf, const S8Stage<GPT>& b) {
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      // A fragments of this group's k-blocks, reused by the 4 strips
      i32x4 af[KBPG][4];
#pragma unroll
      for (int kk = 0; kk < KBPG; ++kk)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int row = a * 16 + r;
          const int chunk = (4 * (gi * KBPG + kk) + g) ^ r;  // row & 15 == r
          af[kk][a] = *(const i32x4*)&As[buf][row * 256 + chunk * 16];
        }
      const int gidx = kt * GPT + gi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        i32x4 acc[4];
#pragma unroll
        for (int kk = 0; kk < KBPG; ++kk) {
          const i32x4 bf = weights_operand_i8(b.code[c][gi * KBPG + kk]);
#pragma unroll
          for (int a = 0; a < 4; ++a)
            acc[a] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                af[kk][a], bf, kk == 0 ? i32x4{0, 0, 0, 0} : acc[a], 0, 0, 0);
        }
        const int n = (st0 + c) * 16 + r;  // accumulator column of this lane
        if (DEBUG_ACC) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tl = a * 16 + 4 * g + i;
              if (tl < nt && c < nst)
                acc_out[((size_t)(t0 + tl) * N + n) * NG + gidx] = acc[a][i] >> 6;
            }
        } else {
          const uint32_t sp = b.sw[c][gi >> 1];
          const float sv =
              half_bits_to_float((uint16_t)((gi & 1) ? (sp >> 16) : (sp & 0xffffu))) * 0.015625f;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              tot[a][c][i] = __builtin_fmaf((float)acc[a][i], sv, tot[a][c][i]);
        }
      }
    }
  };

  // Pipeline, one barrier per k-tile: the activation tile of k-tile kt+1 and
  // the codes/scales of kt+1 are requested before the MFMAs of k-tile kt;
  // then the wave waits for its loads and meets the others at the barrier,
  // after which every wave's part of tile kt+1 is in LDS and nobody reads
  // tile kt's buffer any more. Past the last k-tile the loads repeat it.
  S8Stage<GPT> wA, wB;
  u32x4 av[4];
  if (QPERM) {
    stage_a_direct(0, 0);
  } else {
    load_a_regs(0, av);
  }
  load_w(0, wA);
  if (!QPERM) store_a_regs(0, av);
  // the tile's token scales in LDS for the epilogue (a load per output row
  // there would wait for every store issued before it)
  if (!DEBUG_ACC && tid < kS8BM) sas[tid] = act_scale[t0 + min(tid, nt - 1)];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < KT; kt += 2) {
    const int k1 = min(kt + 1, KT - 1);
    if (QPERM) stage_a_direct(k1, 1); else load_a_regs(k1, av);
    load_w(k1, wB);
    __builtin_amdgcn_sched_barrier(0);
    compute(kt, 0, wA);
    if (!QPERM) store_a_regs(1, av);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 >= KT) break;
    const int k2 = min(kt + 2, KT - 1);
    if (QPERM) stage_a_direct(k2, 0); else load_a_regs(k2, av);
    load_w(k2, wA);
    __builtin_amdgcn_sched_barrier(0);
    compute(kt + 1, 1, wB);
    if (!QPERM) store_a_regs(0, av);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (!DEBUG_ACC) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = a * 16 + 4 * g + i;
        if (tl >= nt) continue;
        const float as = sas[tl];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c < nst) y[(size_t)(t0 + tl) * N + (st0 + c) * 16 + r] = tot[a][c][i] * as;
      }
  }
}

template <bool DEBUG_ACC, bool QPERM>
hipError_t launch_s8_v(const S8Args& a, hipStream_t st) {
  const int NS = a.N / 16;
  dim3 grid((NS + 15) / 16, (a.T + kS8BM - 1) / kS8BM);
  if (a.G == 128)
    hipLaunchKernelGGL((tern_s8_kernel<2, DEBUG_ACC, QPERM>), grid, dim3(256), 0, st, a.q,
                       a.act_scale, a.T, a.K, (const u32x4*)a.codes, a.scales, a.y, a.acc_out, a.N);
  else
    hipLaunchKernelGGL((tern_s8_kernel<4, DEBUG_ACC, QPERM>), grid, dim3(256), 0, st, a.q,
                       a.act_scale, a.T, a.K, (const u32x4*)a.codes, a.scales, a.y, a.acc_out, a.N);
  return (hipError_t)kernel_launched((int)hipGetLastError(),
                                     DEBUG_ACC ? TERN_KERNEL_S8_ACC_EXPORT : TERN_KERNEL_S8_ROW);
}

}  // namespace

template <int NT, int MAXNU>
int launch_quant_perm(int nu, const uint16_t* x, int T, int K, int8_t* q, float* scale, hipStream_t st) {
  switch (nu) {
#define TERN_QP_LAUNCH(NU)                                                                              \
  case NU:                                                                                              \
    if constexpr (NU <= MAXNU)                                                                          \
      hipLaunchKernelGGL((tern_quant_s8_perm_kernel<NU, NT>), dim3(T), dim3(NT), 0, st, x, K, q, scale); \
    break;
    TERN_QP_LAUNCH(1)
    TERN_QP_LAUNCH(2)
    TERN_QP_LAUNCH(3)
    TERN_QP_LAUNCH(4)
    TERN_QP_LAUNCH(5)
    TERN_QP_LAUNCH(6)
    TERN_QP_LAUNCH(7)
    TERN_QP_LAUNCH(8)
#undef TERN_QP_LAUNCH
    default: return (int)hipErrorInvalidValue;
  }
  return kernel_launched((int)hipGetLastError(), TERN_KERNEL_QUANT_S8);
}

int launch_quant_s8(const uint16_t* x, int T, int K, int8_t* q, float* scale, bool operand_order,
                    void* stream) {
  if (T <= 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  // Threads per token. Short batches (fewer tokens than CUs): 1024, for K up
  // to 32768 (two chunks per thread). Long ones: 256 below K = 16384, else
  // 512. Measured at T = 2048 on MI355X: at K = 5120, 256 threads beat 320
  // to 1024 (8.9 against 13.5-18 us); at K = 17408, 512 threads (3 chunks
  // each) ran in 22.1 us against 23.4 with 256 (5 chunks) and 24.1-26.6
  // with 320, 384 and 1024.
  const bool wide_wg = T < 256 && K <= 32768;
  const int nt = wide_wg ? 1024 : K < 16384 ? 256 : 512;
  const int nu = (K / 16 + nt - 1) / nt;  // output chunks per thread
  if (operand_order && nu <= 8) {
    if (nt == 1024) return launch_quant_perm<1024, 2>(nu, x, T, K, q, scale, st);
    if (nt == 512) return launch_quant_perm<512, 8>(nu, x, T, K, q, scale, st);
    return launch_quant_perm<256, 4>(nu, x, T, K, q, scale, st);
  }
  if (operand_order)
    hipLaunchKernelGGL(tern_quant_s8_kernel<true>, dim3(T), dim3(256), 0, (hipStream_t)stream, x, K,
                       q, scale);
  else
    hipLaunchKernelGGL(tern_quant_s8_kernel<false>, dim3(T), dim3(256), 0, (hipStream_t)stream, x,
                       K, q, scale);
  return kernel_launched((int)hipGetLastError(),
                         operand_order ? TERN_KERNEL_QUANT_S8 : TERN_KERNEL_QUANT_S8_ROW);
}

int launch_quant_s8_rot(const uint16_t* x, int T, int K, int8_t* q, float* scale, bool operand_order,
                        void* stream) {
  if (T <= 0) return 0;
  if (K < kRotBlock || K % kRotBlock != 0 || K > kRotMaxK) return (int)hipErrorInvalidValue;
  const int nbw = (K / kRotBlock + 3) / 4;  // blocks per wave
  hipStream_t st = (hipStream_t)stream;
  switch (nbw) {
#define TERN_ROT_LAUNCH(NBW)                                                                             \
  case NBW:                                                                                              \
    if (operand_order)                                                                                   \
      hipLaunchKernelGGL((tern_quant_rot_kernel<NBW, true>), dim3(T), dim3(256), 0, st, x, K, q, scale);  \
    else                                                                                                 \
      hipLaunchKernelGGL((tern_quant_rot_kernel<NBW, false>), dim3(T), dim3(256), 0, st, x, K, q, scale); \
    break;
    TERN_ROT_LAUNCH(1)
    TERN_ROT_LAUNCH(2)
    TERN_ROT_LAUNCH(3)
    TERN_ROT_LAUNCH(4)
    TERN_ROT_LAUNCH(5)
    TERN_ROT_LAUNCH(6)
    TERN_ROT_LAUNCH(7)
    TERN_ROT_LAUNCH(8)
#undef TERN_ROT_LAUNCH
    default: return (int)hipErrorInvalidValue;
  }
  return kernel_launched((int)hipGetLastError(), TERN_KERNEL_QUANT_S8_ROT);
}

int launch_s8(const S8Args& a, const S8Plan& p, void* ws, void* stream) {
  if (a.q_operand_order) return launch_s8_operand_order(a, p, ws, stream);
  if (p.k_parts != 1) return (int)hipErrorInvalidValue;
  hipStream_t st = (hipStream_t)stream;
  const bool dbg = a.acc_out != nullptr;
  if (dbg)
    return (int)(a.q_operand_order ? launch_s8_v<true, true>(a, st) : launch_s8_v<true, false>(a, st));
  return (int)(a.q_operand_order ? launch_s8_v<false, true>(a, st) : launch_s8_v<false, false>(a, st));
}

}  // namespace tern
