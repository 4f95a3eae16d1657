// Chunked-form building blocks shared by the prefill and backward kernels:
// the chunk size, the prepare phase's per-chunk workspace layout, and the
// helpers that move 64-token tiles between LDS, registers and the
// 16x16x32 bf16 MFMA operand layouts (gdn_device.hpp describes the MFMA's
// lane layout).
#pragma once

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int C = kChunk;
constexpr float kLog2e = 1.4426950408889634f;

// Workspace layout of one (batch, head, chunk), in bytes from its start.
// The 64x64 tiles are lower triangular in 16x16 blocks; the scans read
// 32-wide k-blocks at or below the diagonal only, so blocks (0,1) and (2,3)
// hold zeros and rows 0..31, columns 32..63 are never written or read.
constexpr int kWsTh = 0;                    // bf16 [64][64] hi part of T
constexpr int kWsTl = 8192;                 // bf16 [64][64] lo part of T
constexpr int kWsPh = 16384;                // bf16 [64][64] hi part of P
constexpr int kWsPl = 24576;                // bf16 [64][64] lo part of P
// fp32 [4][64] per-token rows: gamma nq (query side, for diag(gamma) Q S^T),
// gamma_C (the chunk's total decay, repeated), gamma nk (key side, for
// V - diag(gamma) K S^T) and e^{g_C - g} nk (for the state update); nq = nk
// = 1 without the input path.
constexpr int kWsG = 32768;
// When the segmented scan forms P itself, the space of P's hi part holds
// fp32 [2][64] exponent rows instead: a_j = log2 gamma_j + log2 nq_j and
// b_i = log2 gamma_i - log2 nk_i, so that P_ji = 2^(a_j - b_i) q~_j . k~_i.
constexpr int kWsAB = kWsPh;
static_assert(kWsG + 4 * 4 * C == kChunkWsFloats * 4, "workspace layout");

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v_t;

// First index of half `half` (0/1) of lane group g4's k-slots in 32-wide
// k-block s: slots 0..3 are kslot_base(s, g4, 0) + 0..3, slots 4..7 are
// kslot_base(s, g4, 1) + 0..3.  These are exactly the rows an accumulator
// tile pair (16s.., 16s+16..) holds in a lane, so accumulators feed B
// operands directly.
__device__ __forceinline__ int kslot_base(int s, int g4, int half) {
  return 32 * s + 16 * half + 4 * g4;
}

// 8 bf16 k-slots of row `row` from a row-major bf16 tile (row stride ld).
__device__ __forceinline__ bf16x8 lds_slots(const bf16* X, int ld, int row,
                                            int s, int g4) {
  const uint2 a = *reinterpret_cast<const uint2*>(&X[row * ld + kslot_base(s, g4, 0)]);
  const uint2 b = *reinterpret_cast<const uint2*>(&X[row * ld + kslot_base(s, g4, 1)]);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Transposing read of a row-major bf16 tile X[row][col] (row stride ld):
// returns, for lane (n = lane % 16), X[r0 + j][c0 + n], j = 0..3.
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element (i % 4) of
// the 4 values read by lane 4 j + i / 4; lane n therefore reads row
// r0 + n / 4, columns c0 + 4 (n % 4) .. + 3.
__device__ __forceinline__ uint2 lds_tr4(const bf16* X, int ld, int r0, int c0,
                                         int n) {
  const bf16* p = &X[(r0 + (n >> 2)) * ld + c0 + 4 * (n & 3)];
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4v_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

// 8 k-slots of k-block s (rows of X are the contraction index) for output
// column c0 + n: X[kslot][c0 + n] via two transposing reads.
__device__ __forceinline__ bf16x8 lds_slots_tr(const bf16* X, int ld, int c0,
                                               int s, int g4, int n) {
  const uint2 a = lds_tr4(X, ld, kslot_base(s, g4, 0), c0, n);
  const uint2 b = lds_tr4(X, ld, kslot_base(s, g4, 1), c0, n);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Accumulator tiles (2s, 2s+1) of a lane as the 8 k-slots of k-block s.
__device__ __forceinline__ floatx8 acc_slots(const floatx4& lo, const floatx4& hi) {
  const floatx8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return x;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return bf16_bits_to_f32(w & 0xFFFFu); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return bf16_bits_to_f32(w >> 16); }

}  // namespace gdn
