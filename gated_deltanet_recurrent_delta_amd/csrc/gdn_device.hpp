// Device helpers shared by the gfx950 kernels of libgdn: bf16 conversions,
// the 16x16x32 bf16 MFMA, split-bf16 operands and 16-lane DPP reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
// 16 bytes as a native vector: register staging in arrays of these stays in
// registers (arrays of the uint4 struct are copied with memcpy and can be
// left in scratch memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return (bf16)x; }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): ~16 significant bits.
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

// Two values rounded to bf16 by one packed conversion: hi2 holds the pair,
// ha and hb the same two roundings as fp32 (exact: a bf16 is the top half
// of an fp32), taken from the packed word by a shift and a mask.
__device__ __forceinline__ void round_pair(float a, float b, uint32_t& hi2,
                                           float& ha, float& hb) {
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const floatx2 p = {a, b};
  hi2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
  ha = __builtin_bit_cast(float, hi2 << 16);
  hb = __builtin_bit_cast(float, hi2 & 0xFFFF0000u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const floatx2 p = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

__device__ __forceinline__ void split8(const floatx8& x, bf16x8& hi,
                                       bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float ha, hb;
    round_pair(x[2 * j], x[2 * j + 1], h[j], ha, hb);
    l[j] = pack_bf16x2(x[2 * j] - ha, x[2 * j + 1] - hb);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

__device__ __forceinline__ void split4(const float* x, bf16x4& hi, bf16x4& lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float ha, hb;
    round_pair(x[2 * j], x[2 * j + 1], h[j], ha, hb);
    l[j] = pack_bf16x2(x[2 * j] - ha, x[2 * j + 1] - hb);
  }
  hi = __builtin_bit_cast(bf16x4, make_uint2(h[0], h[1]));
  lo = __builtin_bit_cast(bf16x4, make_uint2(l[0], l[1]));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const floatx8& x) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                               pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
}

// Load 4 consecutive input elements (bf16 or f32) as float4.
__device__ __forceinline__ float4 load4(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16),
                     bf16_bits_to_f32(u.y & 0xFFFFu), bf16_bits_to_f32(u.y >> 16));
}
__device__ __forceinline__ float4 load4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

__device__ __forceinline__ float load1(const bf16* p) {
  return bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(p));
}
__device__ __forceinline__ float load1(const float* p) { return *p; }

__device__ __forceinline__ void store1(bf16* p, float x) { *p = (bf16)x; }
__device__ __forceinline__ void store1(float* p, float x) { *p = x; }

// Wait until every vector-memory access this wave has issued is complete:
// s_waitcnt vmcnt(0), with the export and LDS/scalar counters left alone
// (simm16 fields on gfx9-family parts: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8).  On gfx950 the vector-memory counter also counts
// stores, so this paces a wave's stores one at a time.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// MFMA: D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16)
//   A: lane l holds row (l % 16), 8 k-values in "slot" order j = 0..7
//   B: lane l holds col (l % 16), the same 8 k-slots
//   D: lane l holds rows 4 * (l / 16) + i, i = 0..3, col (l % 16)
// Only the pairing of A's and B's k-slots matters for the contraction, so a
// kernel may assign any 8 logical k-indices to a lane's slots as long as A
// and B use the same assignment.
// ---------------------------------------------------------------------------

__device__ __forceinline__ floatx4 mfma(const bf16x8& a, const bf16x8& b,
                                        floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// DPP sums over groups of 16 consecutive lanes (result in all 16 lanes)
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xF, 0xF, false));
}

__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: pairs
  x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: quads
  x += dpp<0x141>(x);   // row_half_mirror: lane i <-> 7 - i within 8
  x += dpp<0x140>(x);   // row_mirror: lane i <-> 15 - i within 16
  return x;
}

}  // namespace gdn
