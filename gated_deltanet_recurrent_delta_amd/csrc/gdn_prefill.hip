// Chunked prefill of the gated delta rule on gfx950.
//
// The token recurrence (decay, predict with the decayed state, delta write,
// read the new state; "On State Reduction in Linear Attention", paper Sec. 2.1,
// Eq. (2) with gated decay, and "Linear Attention Architectures", paper Sec. 3.3)
// is evaluated 64 tokens at a time.  Unrolling it inside a chunk of C tokens
// with incoming state S, g = cumsum(log alpha) (inclusive, within the
// chunk), gamma_j = e^{g_j}:
//
//   u_j = beta_j (v_j - alpha_j S_{j-1} k_j)  satisfies the unit lower
//   triangular system (I + A) U = diag(beta) (V - diag(gamma) K S^T) with
//   A_ji = beta_j e^{g_j - g_i} k_j.k_i for i < j, so
//
//     U   = T diag(beta) (V - diag(gamma) K S^T),   T = (I + A)^{-1}
//     O   = diag(gamma) Q S^T + P U,  P_ji = e^{g_j - g_i} q_j.k_i (i <= j)
//     S' = gamma_C S + U^T diag(e^{g_C - g}) K
//
// This is an exact re-association of the sequential recurrence.  The
// workspace holds T diag(beta) (so the scan forms V - diag(gamma) K S^T and
// one product), and the optional input path (keep a per-head subset of the
// query/key channels, renormalise over the kept channels, scale the query;
// "On State Reduction in Linear Attention", paper Sec. 3.2-3.3) enters only as
// per-token factors: with q_j = nq_j q~_j and k_j = nk_j k~_j (q~, k~ the
// kept raw channels, nq_j = scale / |q~_j|, nk_j = 1 / |k~_j|), the raw
// rows stay exact MFMA operands and nk, nq are folded into A, P and the
// per-token decay rows the scan reads (gamma nq, gamma nk, e^{g_C - g} nk).
//
// The kernels:
//  * prepare_kernel -- one wave per (batch, head, chunk), fully parallel.
//    K and Q are read once from HBM straight into MFMA operand registers
//    (with a channel subset: the kept channels, also written out as the
//    gathered copy the scan reads);
//    the lower 16x16 tiles of K K^T and Q K^T run on bf16 MFMA; the decay
//    factors are exp2 of differences of the scaled prefix sums (never of a
//    single prefix sum, which can underflow); T is inverted in fp32 (the four
//    16x16 diagonal blocks by forward substitution, one lane per column, then
//    the off-diagonal blocks level by level).  T and P are written as bf16
//    hi/lo tiles ready to be copied into LDS.
//  * scan_kernel -- one workgroup per (batch, head, 16 NW state rows).  The
//    rows of the state evolve independently ("On State Reduction in Linear
//    Attention", paper Sec. 3.1), so each wave owns 16 rows and runs the whole
//    chunk step for them in registers: the MFMA accumulator tiles of S, Y, Z
//    and U are fed back as B operands without an LDS round trip (a lane's 8
//    k-slots are the two 4-row runs it holds in the accumulator layout).
//    The waves share one LDS copy of the chunk's K, Q, T, P and V tiles,
//    staged with 16-byte copies from registers that were prefetched while
//    the previous chunk computed; K^T and V^T operands come from the
//    row-major tiles through the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16), so no transposed copy is kept.
//    Products that touch the state use split-bf16 operands (x = hi + lo, two
//    MFMAs when the other operand is an exact bf16 input, three otherwise)
//    with fp32 accumulation; outputs stored in bf16 use single-pass products.
//  * scan_wide_kernel, segment_combine_kernel, segment_correct_kernel --
//    the segmented scan for few heads and long sequences (bf16 in and out):
//    every segment runs from a zero state together with transition rows
//    that give its affine map, the segment states are chained, and the
//    outputs of later segments are corrected (see SegArgs).
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "gdn_tiles.hpp"

namespace gdn {

namespace {

// (chunk size, workspace layout and the MFMA tile helpers: gdn_tiles.hpp)

// 8 consecutive inputs as bf16 hi (and lo when the input is fp32).
__device__ __forceinline__ void load_row8(const bf16* p, bf16x8& hi, bf16x8& lo) {
  hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  (void)lo;
}
__device__ __forceinline__ void load_row8(const float* p, bf16x8& hi, bf16x8& lo) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const floatx8 x = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  split8(x, hi, lo);
}

// 8 inputs as fp32: consecutive, or gathered at channel indices ci.
__device__ __forceinline__ void ld8(const bf16* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16lo(w[j]);
    x[2 * j + 1] = bf16hi(w[j]);
  }
}
__device__ __forceinline__ void ld8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void ld8_gather(const bf16* row, const int (&ci)[8], float (&x)[8]) {
  const uint16_t* r = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = bf16_bits_to_f32(r[ci[e]]);
}
__device__ __forceinline__ void ld8_gather(const float* row, const int (&ci)[8], float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = row[ci[e]];
}
// 8 values stored exactly in the input type
__device__ __forceinline__ void st8(bf16* p, const float (&x)[8]) {
  const floatx8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  *reinterpret_cast<bf16x8*>(p) = to_bf16x8(v);      // exact: x holds bf16 values
}
__device__ __forceinline__ void st8(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
// MFMA operands of 8 input values: bf16 inputs exactly, fp32 as hi + lo.
template <bool SPLIT>
__device__ __forceinline__ void pack8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  const floatx8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  if constexpr (SPLIT) split8(v, hi, lo);
  else hi = to_bf16x8(v);
}
__device__ __forceinline__ float sumsq8(const float (&x)[8]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += x[e] * x[e];
  return s;
}
__device__ __forceinline__ float sumsq8(const bf16x8& x) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = (float)x[e];
    s += f * f;
  }
  return s;
}
// 1 / |x| from |x|^2 (0 for a zero vector), or 1 without normalisation.
__device__ __forceinline__ float inv_norm(float ss, int l2norm) {
  return l2norm ? (ss > 0.f ? 1.f / sqrtf(ss) : 0.f) : 1.f;
}

}  // namespace

// ===========================================================================
// prepare: one wave per chunk
// ===========================================================================

// Index of the strictly lower 16x16 tile (mi > ni) among the six of a 64x64
// matrix: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
__device__ __forceinline__ constexpr int lower_tile(int mi, int ni) {
  return mi * (mi - 1) / 2 + ni;
}

// The chunk products are formed in row orientation: for a 16x16 tile
// (mi, ni) lane (n, g4) holds element [16 mi + n][16 ni + 4 g4 + e],
// e = 0..3 (the MFMA computes K_ni K_mi^T, whose lane layout is that of the
// transposed tile).  A lane thus holds four consecutive columns of one row:
// P leaves with one 8-byte store per tile, and the off-diagonal tiles of A
// are, as they stand, the A operand of the fp32 MFMAs that build T.  Only T
// (with A's diagonal blocks before it) passes through LDS, 17.9 KB per
// wave, so eight waves share a CU and one wave's loads overlap another's
// arithmetic.
// NOP: the segmented scan forms P itself from the staged K and Q tiles; the
// kernel then skips P (and, without the input path's norms or gather, the
// query rows) and writes the two exponent rows that scan needs instead.
// The bf16 channel-pick instance at DK = 64 is held to two waves per SIMD:
// unbounded it took 258 registers (one wave per SIMD), bounded it fits 256
// without spilling, and the batched prefill from 128-wide rows went from
// 345-352 to 327 us (B=8, T=4096, H=16).
template <int DK, typename TIn, bool GATHER, bool NOP>
__global__ __launch_bounds__(64, (GATHER && DK == 64 && !std::is_same<TIn, float>::value) ? 2 : 1)
void prepare_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ ws, int T, int H, int nchunks, int write_pl, QkArgs qa) {
  constexpr bool SPLIT = std::is_same<TIn, float>::value;  // inputs not bf16
  constexpr int NKB = DK / 32;
  constexpr int LDA = C + 4;            // fp32 row stride of the T tile
  __shared__ __attribute__((aligned(16))) float Ts[C * LDA];   // A's diagonal blocks, then T
  __shared__ __attribute__((aligned(16))) float g2s[C];
  __shared__ __attribute__((aligned(16))) float bs[C];
  __shared__ __attribute__((aligned(16))) float nks[C];       // 1 / |k~_j| (or 1)
  __shared__ __attribute__((aligned(16))) float nqs[C];       // scale / |q~_j| (or scale)

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = chunk * C;
  const int nvalid = min(C, T - t0);
  const int lane = threadIdx.x, n = lane & 15, g4 = lane >> 4;
  char* wsc = reinterpret_cast<char*>(ws) +
              ((size_t)(b * H + h) * nchunks + chunk) * kChunkWsFloats * 4;

  // 1. gates of the chunk first (vector-memory results return in order, so
  //    the prefix sum below does not wait for the K/Q tiles), then K and Q
  //    rows 16 t + n, k-slots 32 s + 8 g4 .. + 7, straight from HBM: the
  //    row itself, or (GATHER) the kept channels chan[h][32 s + 8 g4 + e] of
  //    the dk_in-wide row, which are also written out as the gathered copy
  //    the scan reads.  ssk/ssq: this lane's part of |k~|^2 and |q~|^2.
  float a_in = 1.f, be = 0.f;               // padding tokens: identity step
  if (lane < nvalid) {
    const size_t gi = ((size_t)b * T + t0 + lane) * H + h;
    a_in = alpha[gi];
    be = beta[gi];
  }
  int ci[GATHER ? NKB : 1][8];
  if constexpr (GATHER) {
#pragma unroll
    for (int s = 0; s < NKB; ++s) {
      const int4 c0 = *reinterpret_cast<const int4*>(qa.chan + (size_t)h * DK + 32 * s + 8 * g4);
      const int4 c1 = *reinterpret_cast<const int4*>(qa.chan + (size_t)h * DK + 32 * s + 8 * g4 + 4);
      ci[s][0] = c0.x; ci[s][1] = c0.y; ci[s][2] = c0.z; ci[s][3] = c0.w;
      ci[s][4] = c1.x; ci[s][5] = c1.y; ci[s][6] = c1.z; ci[s][7] = c1.w;
      // an index outside the row is clamped into it: never an out-of-bounds read
#pragma unroll
      for (int e = 0; e < 8; ++e) ci[s][e] = min(max(ci[s][e], 0), qa.dk_in - 1);
    }
  }
  const int ldin = GATHER ? qa.dk_in : DK;  // row width of q, k in memory
  TIn* kg = nullptr;                        // GATHER: the gathered copy of k, then q
  TIn* qg = nullptr;
  if constexpr (GATHER) {
    kg = static_cast<TIn*>(qa.qk_out);
    qg = kg + (size_t)gridDim.z * T * H * DK;
  }
  bf16x8 Kh[4][NKB], Kl[4][NKB], Qh[4][NKB], Ql[4][NKB];
  float ssk[4], ssq[4];
  // The pruned width from bf16 rows 128 wide (16-byte aligned): every raw
  // row is read whole with 16-byte loads, staged in LDS (the space of the T
  // tile, not in use yet) and the kept channels are picked there; other
  // widths read the kept channels one element at a time.
  constexpr bool STAGE = GATHER && !SPLIT && DK == 64;
  constexpr int LDR = 136;                   // staged row stride (one 16-byte pad unit)
  static_assert(C * LDR * 2 <= C * LDA * 4, "staged rows fit in the T tile");
  bool staged = false;
  uint4 rk[STAGE ? 16 : 1], rq[STAGE ? 16 : 1];   // lane: unit n of rows 4 j + g4
  if constexpr (STAGE) {
    staged = qa.dk_in == 128 && ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) & 15) == 0;
    if (staged) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = 4 * j + g4;
        rk[j] = rq[j] = make_uint4(0u, 0u, 0u, 0u);
        if (row < nvalid) {
          const size_t off = (((size_t)b * T + t0 + row) * H + h) * 128 + 8 * n;
          rk[j] = *reinterpret_cast<const uint4*>(k + off);
          rq[j] = *reinterpret_cast<const uint4*>(q + off);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 4 && !staged; ++t) {
    const int c = 16 * t + n;
    const size_t row = ((size_t)b * T + t0 + c) * H + h;           // token row
    ssk[t] = ssq[t] = 0.f;
#pragma unroll
    for (int s = 0; s < NKB; ++s) {
      const bf16x8 z = {};
      Kh[t][s] = Kl[t][s] = Qh[t][s] = Ql[t][s] = z;
      if (c < nvalid) {
        const size_t off = row * DK + 32 * s + 8 * g4;              // kept-width layout
        if constexpr (GATHER || SPLIT) {
          float xk[8], xq[8];
          if constexpr (GATHER) {
            ld8_gather(k + row * ldin, ci[s], xk);
            ld8_gather(q + row * ldin, ci[s], xq);
            st8(kg + off, xk);
            st8(qg + off, xq);
          } else {
            ld8(k + off, xk);
            ld8(q + off, xq);
          }
          pack8<SPLIT>(xk, Kh[t][s], Kl[t][s]);
          pack8<SPLIT>(xq, Qh[t][s], Ql[t][s]);
          ssk[t] += sumsq8(xk);
          ssq[t] += sumsq8(xq);
        } else {
          Kh[t][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(k + off));
          if (!NOP || qa.l2norm)             // the query rows feed P or |q|
            Qh[t][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + off));
        }
      }
    }
  }

  // 2. gates: inclusive prefix sum of log alpha inside the chunk (lane =
  //    token j); the rows that need the norms are written in step 2b
  float gam, dec, gamC;
  {
    float g = logf(a_in);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(g, off, 64);
      if (lane >= off) g += y;
    }
    const float glast = __shfl(g, 63, 64);
    g2s[lane] = g * kLog2e;
    bs[lane] = be;
    gam = expf(g);
    dec = expf(glast - g);
    gamC = expf(glast);
  }

  // 1b. staged rows: pick the kept channels from LDS (after the gate prefix
  //     sum, which then does not wait for the rows)
  if constexpr (STAGE) {
    if (staged) {
      bf16* stg = reinterpret_cast<bf16*>(Ts);
      auto pick = [&](const uint4 (&raw)[16], bf16x8 (&X)[4][NKB], float (&ss)[4], bf16* copy) {
        __syncthreads();                       // earlier reads of the staging area are done
#pragma unroll
        for (int j = 0; j < 16; ++j)
          *reinterpret_cast<uint4*>(&stg[(4 * j + g4) * LDR + 8 * n]) = raw[j];
        __syncthreads();
        const uint16_t* s16 = reinterpret_cast<const uint16_t*>(stg);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = 16 * t + n;
          ss[t] = 0.f;
#pragma unroll
          for (int s = 0; s < NKB; ++s) {
            uint32_t w[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
              w[p] = (uint32_t)s16[c * LDR + ci[s][2 * p]] |
                     ((uint32_t)s16[c * LDR + ci[s][2 * p + 1]] << 16);
            X[t][s] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            if (c < nvalid)
              *reinterpret_cast<uint4*>(copy + (((size_t)b * T + t0 + c) * H + h) * DK +
                                        32 * s + 8 * g4) = make_uint4(w[0], w[1], w[2], w[3]);
            ss[t] += sumsq8(X[t][s]);
          }
        }
      };
      pick(rk, Kh, ssk, kg);
      pick(rq, Qh, ssq, qg);
    }
  }

  // 2b. per-token factors of the input path: the four lanes of a token
  //     (g4 = 0..3) hold its k-slots; 1 and qscale without normalisation
  {
    if constexpr (!GATHER && !SPLIT) {
      if (qa.l2norm) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int s = 0; s < NKB; ++s) {
            ssk[t] += sumsq8(Kh[t][s]);
            ssq[t] += sumsq8(Qh[t][s]);
          }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float sk = ssk[t], sq = ssq[t];
      if (qa.l2norm) {
        sk += __shfl_xor(sk, 16, 64);
        sk += __shfl_xor(sk, 32, 64);
        sq += __shfl_xor(sq, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
      }
      if (g4 == 0) {
        nks[16 * t + n] = inv_norm(sk, qa.l2norm);
        nqs[16 * t + n] = inv_norm(sq, qa.l2norm) * qa.qscale;
      }
    }
  }
  __syncthreads();
  {
    float* Gw = reinterpret_cast<float*>(wsc + kWsG);
    const float nk = nks[lane], nq = nqs[lane];
    Gw[lane] = gam * nq;
    Gw[C + lane] = gamC;
    Gw[2 * C + lane] = gam * nk;
    Gw[3 * C + lane] = dec * nk;
    if constexpr (NOP) {
      // P_ji = 2^(a_j - b_i) q~_j . k~_i (i <= j) with a_j = log2 gamma_j
      // + log2 nq_j and b_i = log2 gamma_i - log2 nk_i, over the staged rows
      float* Ab = reinterpret_cast<float*>(wsc + kWsAB);
      Ab[lane] = g2s[lane] + __builtin_amdgcn_logf(nq);
      Ab[C + lane] = g2s[lane] - __builtin_amdgcn_logf(nk);
    }
  }

  // 3. lower tiles of A (decay- and beta-weighted K K^T, strictly lower) and
  //    of P (decay-masked Q K^T), row orientation; P straight to the
  //    workspace, with zeros in its upper tiles (0,1) and (2,3).
  floatx4 Ao[6];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int j = 16 * mi + n;                // row of this lane
    const float gj = g2s[j], bj = bs[j] * nks[j], qj = nqs[j];
#pragma unroll
    for (int ni = 0; ni <= mi; ++ni) {
      floatx4 ak = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKB; ++s) {
        ak = mfma(Kh[ni][s], Kh[mi][s], ak);
        if constexpr (!NOP) aq = mfma(Kh[ni][s], Qh[mi][s], aq);
        if constexpr (SPLIT) {
          ak = mfma(Kl[ni][s], Kh[mi][s], ak);
          ak = mfma(Kh[ni][s], Kl[mi][s], ak);
          if constexpr (!NOP) {
            aq = mfma(Kl[ni][s], Qh[mi][s], aq);
            aq = mfma(Kh[ni][s], Ql[mi][s], aq);
          }
        }
      }
      const int i0 = 16 * ni + 4 * g4;        // first column of this lane
      const float4 gi4 = *reinterpret_cast<const float4*>(&g2s[i0]);
      const float gi[4] = {gi4.x, gi4.y, gi4.z, gi4.w};
      const float4 nk4 = *reinterpret_cast<const float4*>(&nks[i0]);
      const float nki[4] = {nk4.x, nk4.y, nk4.z, nk4.w};
      float a[4], p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        const float decay = (i <= j) ? __builtin_amdgcn_exp2f(gj - gi[e]) * nki[e] : 0.f;
        a[e] = (i < j) ? bj * decay * ak[e] : 0.f;
        p[e] = qj * decay * aq[e];
      }
      if constexpr (!NOP) {
        bf16x4 ph, pl;
        split4(p, ph, pl);
        *reinterpret_cast<bf16x4*>(wsc + kWsPh + (j * C + i0) * 2) = ph;
        if (write_pl) *reinterpret_cast<bf16x4*>(wsc + kWsPl + (j * C + i0) * 2) = pl;
      }
      if (ni == mi)
        *reinterpret_cast<float4*>(&Ts[j * LDA + i0]) = make_float4(a[0], a[1], a[2], a[3]);
      else
        Ao[lower_tile(mi, ni)] = floatx4{a[0], a[1], a[2], a[3]};
    }
    // zeros only in the upper tile that shares a 32-wide k-block with the
    // diagonal one ((0,1) and (2,3)): the scans read k-blocks s <= ct / 2
    // only, so rows 0..31 never read columns 32..63, which stay unwritten
    const bf16x4 zero4 = {};
    if (!NOP && (mi & 1) == 0) {
      const int ni = mi + 1;
      *reinterpret_cast<bf16x4*>(wsc + kWsPh + (j * C + 16 * ni + 4 * g4) * 2) = zero4;
      if (write_pl) *reinterpret_cast<bf16x4*>(wsc + kWsPl + (j * C + 16 * ni + 4 * g4) * 2) = zero4;
    }
  }
  __syncthreads();

  // 4. T = (I + A)^{-1}.  Diagonal blocks by forward substitution, lane
  //    (block g4, column n), reading A's diagonal block from Ts and then
  //    overwriting it with T's.
  {
    const int base = 16 * g4, c = n;
    float tcol[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float acc0 = (j == c) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
      for (int i = 0; i < j; i += 2) {
        acc0 -= Ts[(base + j) * LDA + base + i] * tcol[i];
        if (i + 1 < j) acc1 -= Ts[(base + j) * LDA + base + i + 1] * tcol[i + 1];
      }
      tcol[j] = acc0 + acc1;
    }
    __syncthreads();                          // every lane has read its block of A
#pragma unroll
    for (int j = 0; j < 16; ++j) Ts[(base + j) * LDA + base + c] = tcol[j];
    // zero the upper blocks of T that are stored: (0,1) and (2,3)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
      if (bj > g4 && (bj >> 1) == (g4 >> 1))
#pragma unroll
        for (int j = 0; j < 16; ++j) Ts[(base + j) * LDA + 16 * bj + c] = 0.f;
  }
  __syncthreads();
  // Off-diagonal blocks, nearest the diagonal first:
  //   T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj   (i > j, 16x16 blocks)
  // on fp32 MFMA (16x16x4, exact fp32 products).  A step kk of a 16x16x16
  // product contracts over k = 4 g4 + kk: the row-oriented A tiles supply
  // the A operand as they are, and the accumulator of the first product
  // (lane holds rows 4 g4 + i) is the B operand of the second one.
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
#pragma unroll
    for (int bj = 0; bj + dist < 4; ++bj) {
      const int bi = bj + dist;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bk = bj; bk < bi; ++bk) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float y = Ts[(16 * bk + 4 * g4 + kk) * LDA + 16 * bj + n];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ao[lower_tile(bi, bk)][kk], y, acc, 0, 0, 0);
        }
      }
      floatx4 out = {0.f, 0.f, 0.f, 0.f};
      const float4 tii = *reinterpret_cast<const float4*>(&Ts[(16 * bi + n) * LDA + 16 * bi + 4 * g4]);
      const float tv[4] = {tii.x, tii.y, tii.z, tii.w};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        out = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[kk], acc[kk], out, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) Ts[(16 * bi + 4 * g4 + i) * LDA + 16 * bj + n] = -out[i];
    }
    __syncthreads();
  }

  // 5. T diag(beta) -> workspace as bf16 hi/lo (rows 0..31, columns
  //    32..63 are never read and stay unwritten)
  for (int e = lane; e < C * C / 8; e += 64) {
    const int j = (8 * e) / C, i0 = (8 * e) % C;
    if (j < C / 2 && i0 >= C / 2) continue;
    const float4 a0 = *reinterpret_cast<const float4*>(&Ts[j * LDA + i0]);
    const float4 a1 = *reinterpret_cast<const float4*>(&Ts[j * LDA + i0 + 4]);
    const float4 b0 = *reinterpret_cast<const float4*>(&bs[i0]);
    const float4 b1 = *reinterpret_cast<const float4*>(&bs[i0 + 4]);
    const floatx8 x = {a0.x * b0.x, a0.y * b0.y, a0.z * b0.z, a0.w * b0.w,
                       a1.x * b1.x, a1.y * b1.y, a1.z * b1.z, a1.w * b1.w};
    bf16x8 hi, lo;
    split8(x, hi, lo);
    *reinterpret_cast<bf16x8*>(wsc + kWsTh + (j * C + i0) * 2) = hi;
    *reinterpret_cast<bf16x8*>(wsc + kWsTl + (j * C + i0) * 2) = lo;
    if (qa.t_out != nullptr) {            // T itself, for the backward pass
      char* tu = static_cast<char*>(qa.t_out) + ((size_t)(b * H + h) * nchunks + chunk) * kTuBytes;
      const floatx8 t = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      split8(t, hi, lo);
      *reinterpret_cast<bf16x8*>(tu + (j * C + i0) * 2) = hi;
      *reinterpret_cast<bf16x8*>(tu + C * C * 2 + (j * C + i0) * 2) = lo;
    }
  }
}

// ===========================================================================
// scan
// ===========================================================================

// Per-thread register staging of one chunk for NT threads.  NTP of the four
// bf16 64x64 tiles (T hi, T lo, P hi, P lo) are staged: P lo only feeds
// fp32 outputs.  U16: the 16-byte unit type (the state-storing sweep takes
// the native vector, with which its staging stays out of scratch memory).
template <int DK, typename TIn, int NT, int ROWS, int NTP, typename U16>
struct Stage {
  static constexpr int UNITS_K = C * DK * (int)sizeof(TIn) / 16 / NT;    // 16B units
  static constexpr int UNITS_TP = NTP * C * C * 2 / 16 / NT;             // T, P tiles
  static constexpr int UNITS_V = C * ROWS * (int)sizeof(TIn) / 16 / NT;  // V rows of the WG
  static_assert(UNITS_K * NT * 16 == C * DK * (int)sizeof(TIn), "K staging");
  static_assert(UNITS_TP * NT * 16 == NTP * C * C * 2, "T/P staging");
  static_assert(UNITS_V * NT * 16 == C * ROWS * (int)sizeof(TIn), "V staging");
  U16 k[UNITS_K];
  U16 q[UNITS_K];
  U16 tp[UNITS_TP];
  U16 v[UNITS_V];
  float g;
};

// MINW: waves per SIMD the kernel is compiled for.  MINW = 2 lets two
// workgroups share a CU so that one hides the other's LDS and memory
// latency, at the price of a tighter register budget; it is used when the
// grid has more workgroups than the GPU has CUs.
// SC: the backward pass's forward sweep: no outputs; the state at the
// start of every chunk goes to Sc ([B*H][nchunks][DV][DK] fp32).
template <int DK, typename TIn, typename TOut, int NW, int MINW, bool SC = false>
__global__ __launch_bounds__(64 * NW, MINW) void scan_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* S0, TOut* __restrict__ o,
    float* ST, const float* __restrict__ ws, int T, int H, int DV,
    int nchunks, int nblocks, float* __restrict__ Sc) {
  constexpr bool KEXACT = std::is_same<TIn, bf16>::value;   // q, k, v exact in bf16
  constexpr bool OPREC = std::is_same<TOut, float>::value;  // o stored in fp32
  constexpr int NT = 64 * NW;           // threads
  constexpr int ROWS = 16 * NW;         // state rows of the workgroup
  constexpr int LDK = DK + 8;           // bf16 stride of the K / Q tiles
  constexpr int LDT = C + 8;            // bf16 stride of the T / P tiles
  constexpr int LDV = 16 + 8;           // bf16 stride of a wave's V block [c][16 r]
  constexpr int VBLK = C * LDV;         // elements per wave block
  constexpr int NDT = DK / 16;          // d-tiles of a 16-row state slice
  constexpr int NKB = DK / 32;          // 32-wide k-blocks over d
  constexpr int EPU = 16 / (int)sizeof(TIn);    // input elements per 16B unit
  constexpr int UPR = DK / EPU;                 // 16B units per K/Q row
  constexpr int VUPR = ROWS / EPU;              // 16B units per V row
  constexpr int NTP = OPREC ? 4 : 3;    // staged T/P tiles
  using U16 = typename std::conditional<SC, u32x4, uint4>::type;
  using St = Stage<DK, TIn, NT, ROWS, NTP, U16>;

  __shared__ __attribute__((aligned(16))) bf16 Khs[C * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Kls[KEXACT ? 8 : C * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Qhs[C * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Qls[KEXACT ? 8 : C * LDK];
  __shared__ __attribute__((aligned(16))) bf16 TPs[NTP][C * LDT];   // Th, Tl, Ph[, Pl]
  // V tile blocked by wave (block w = rows 16 w .. 16 w + 15 of the group);
  // once a wave has formed Z, its block is reused to stage its O^T tile.
  __shared__ __attribute__((aligned(16))) bf16 Vhs[NW * VBLK];
  __shared__ __attribute__((aligned(16))) bf16 Vls[KEXACT ? 8 : NW * VBLK];
  __shared__ __attribute__((aligned(16))) float Gs[4 * C];
  // per-wave O^T staging [16 r][C c] for 16-byte output stores (bf16 o)
  constexpr int LDO = C + 8;
  static_assert(16 * LDO <= VBLK, "O^T staging fits in a wave's V block");
  const bf16* Ths = TPs[0];
  const bf16* Tls = TPs[1];
  const bf16* Phs = TPs[2];
  const bf16* Pls = TPs[NTP - 1];       // (read only for fp32 outputs)

  // workgroup -> (head, row group); the row groups of a head are placed on
  // one XCD (workgroups are dealt to the 8 XCDs round-robin) so they share
  // that XCD's L2 copy of the chunk tiles.
  int lin = blockIdx.x;
  if ((nblocks & 7) == 0) lin = (lin & 7) * (nblocks >> 3) + (lin >> 3);
  const int NRG = DV / ROWS;
  const int bh = lin / NRG, rg = lin - bh * NRG;
  const int b = bh / H, h = bh - b * H;
  const int r0 = rg * ROWS;                 // first row of the group

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int rw = 16 * w;                    // this wave's rows within the group

  // Token rows of this sequence start at k_seq / q_seq / v_seq; one token
  // is H * DK (H * DV) elements further.
  const TIn* k_seq = k + ((size_t)b * T * H + h) * DK;
  const TIn* q_seq = q + ((size_t)b * T * H + h) * DK;
  const TIn* v_seq = v + ((size_t)b * T * H + h) * DV + r0;
  const size_t tok_k = (size_t)H * DK, tok_v = (size_t)H * DV;
  // Rows past the end of the sequence load the last valid row (always in
  // bounds); commit_stage zeroes them.  Nothing reads the loaded registers
  // before the commit, so the loads stay in flight while the previous chunk
  // computes.
  auto load_stage = [&](St& st, int chunk) {
    const int t0 = chunk * C;
    const int nvalid = min(C, T - t0);
#pragma unroll
    for (int i = 0; i < St::UNITS_K; ++i) {
      const int u = tid + NT * i;
      const int c = u / UPR, cu = u - c * UPR;
      const size_t off = (size_t)(t0 + min(c, nvalid - 1)) * tok_k + cu * EPU;
      st.k[i] = *reinterpret_cast<const U16*>(k_seq + off);
      if constexpr (!SC) st.q[i] = *reinterpret_cast<const U16*>(q_seq + off);
    }
#pragma unroll
    for (int i = 0; i < St::UNITS_V; ++i) {
      const int u = tid + NT * i;
      const int c = u / VUPR, cu = u - c * VUPR;
      st.v[i] = *reinterpret_cast<const U16*>(
          v_seq + (size_t)(t0 + min(c, nvalid - 1)) * tok_v + cu * EPU);
    }
    const char* wsc = reinterpret_cast<const char*>(ws) +
                      ((size_t)bh * nchunks + chunk) * kChunkWsFloats * 4;
#pragma unroll
    for (int i = 0; i < St::UNITS_TP; ++i)
      st.tp[i] = *reinterpret_cast<const U16*>(wsc + 16 * (tid + NT * i));
    st.g = (tid < 4 * C) ? reinterpret_cast<const float*>(wsc + kWsG)[tid] : 0.f;
  };

  auto commit_stage = [&](const St& st, int nvalid) {
#pragma unroll
    for (int i = 0; i < St::UNITS_K; ++i) {
      const int u = tid + NT * i;
      const int c = u / UPR, d0 = (u - c * UPR) * EPU;
      const uint32_t mk = c < nvalid ? 0xFFFFFFFFu : 0u;   // (a select on uint4 spills)
      const uint4 kx = make_uint4(st.k[i].x & mk, st.k[i].y & mk, st.k[i].z & mk, st.k[i].w & mk);
      const uint4 qx = SC ? kx : make_uint4(st.q[i].x & mk, st.q[i].y & mk, st.q[i].z & mk, st.q[i].w & mk);
      if constexpr (KEXACT) {
        *reinterpret_cast<uint4*>(&Khs[c * LDK + d0]) = kx;
        if constexpr (!SC) *reinterpret_cast<uint4*>(&Qhs[c * LDK + d0]) = qx;
      } else {
        const float4 kf = __builtin_bit_cast(float4, kx);
        const float4 qf = __builtin_bit_cast(float4, qx);
        const float kx[4] = {kf.x, kf.y, kf.z, kf.w};
        const float qx[4] = {qf.x, qf.y, qf.z, qf.w};
        bf16x4 kh, kl, qh, ql;
        split4(kx, kh, kl);
        split4(qx, qh, ql);
        *reinterpret_cast<bf16x4*>(&Khs[c * LDK + d0]) = kh;
        *reinterpret_cast<bf16x4*>(&Kls[c * LDK + d0]) = kl;
        *reinterpret_cast<bf16x4*>(&Qhs[c * LDK + d0]) = qh;
        *reinterpret_cast<bf16x4*>(&Qls[c * LDK + d0]) = ql;
      }
    }
#pragma unroll
    for (int i = 0; i < St::UNITS_TP; ++i) {
      const int u = tid + NT * i;             // 16B unit of [4][64][64] bf16
      const int m = u >> 9, rem = u & 511;    // 512 units per 64x64 matrix (m < NTP)
      const int j = rem >> 3, i0 = (rem & 7) * 8;
      *reinterpret_cast<U16*>(&TPs[m][j * LDT + i0]) = st.tp[i];
    }
#pragma unroll
    for (int i = 0; i < St::UNITS_V; ++i) {
      const int u = tid + NT * i;
      const int c = u / VUPR, rr = (u - c * VUPR) * EPU;
      const int vb = (rr >> 4) * VBLK + c * LDV + (rr & 15);   // wave block, row c
      const uint32_t mv = c < nvalid ? 0xFFFFFFFFu : 0u;
      const uint4 vx = make_uint4(st.v[i].x & mv, st.v[i].y & mv, st.v[i].z & mv, st.v[i].w & mv);
      if constexpr (KEXACT) {
        *reinterpret_cast<uint4*>(&Vhs[vb]) = vx;
      } else {
        const float4 vf = __builtin_bit_cast(float4, vx);
        const float vx[4] = {vf.x, vf.y, vf.z, vf.w};
        bf16x4 vh, vl;
        split4(vx, vh, vl);
        *reinterpret_cast<bf16x4*>(&Vhs[vb]) = vh;
        *reinterpret_cast<bf16x4*>(&Vls[vb]) = vl;
      }
    }
    if (tid < 4 * C) Gs[tid] = st.g;
  };

  // ---- carried state of this wave: S^T tiles, lane holds
  //      S^T[d = 16 dt + 4 g4 + i][r = n]  (i = 0..3) ----
  floatx4 S[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    if (S0 != nullptr) {
      const float4 x = *reinterpret_cast<const float4*>(
          S0 + ((size_t)bh * DV + r0 + rw + n) * DK + 16 * dt + 4 * g4);
      S[dt] = floatx4{x.x, x.y, x.z, x.w};
    } else {
      S[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // obase + t * ostride is token t's first element of this wave's 16 rows.
  TOut* const obase = o + ((size_t)b * T * H + h) * DV + r0 + rw;
  const size_t ostride = (size_t)H * DV;

  St st;
  load_stage(st, 0);

  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int t0 = chunk * C;
    const int nvalid = min(C, T - t0);
    __syncthreads();                   // everyone is done with the last tiles
    commit_stage(st, nvalid);
    __syncthreads();
    if (chunk + 1 < nchunks) load_stage(st, chunk + 1);   // prefetch
    if constexpr (SC) {
      const size_t srow = ((size_t)bh * nchunks + chunk) * DV + r0 + rw + n;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<float4*>(Sc + srow * DK + 16 * dt + 4 * g4) =
            make_float4(S[dt][0], S[dt][1], S[dt][2], S[dt][3]);
    }

    // split the state into bf16 hi/lo B operands, one per 32-wide k-block
    bf16x8 Sh[NKB], Sl[NKB];
#pragma unroll
    for (int s = 0; s < NKB; ++s) split8(acc_slots(S[2 * s], S[2 * s + 1]), Sh[s], Sl[s]);

    // ---- Y = K S^T and Q S^T  (c-tile ct: rows c = 16 ct + 4 g4 + i,
    //      col r = n); both contract the state over d ----
    floatx4 Y[4], OQ[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f}, accq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKB; ++s) {
        const bf16x8 kh = lds_slots(Khs, LDK, 16 * ct + n, s, g4);
        const bf16x8 qh = lds_slots(Qhs, LDK, 16 * ct + n, s, g4);
        acc = mfma(kh, Sh[s], acc);
        acc = mfma(kh, Sl[s], acc);
        if constexpr (!KEXACT) acc = mfma(lds_slots(Kls, LDK, 16 * ct + n, s, g4), Sh[s], acc);
        if constexpr (SC) continue;
        accq = mfma(qh, Sh[s], accq);
        if constexpr (OPREC) {
          accq = mfma(qh, Sl[s], accq);
          if constexpr (!KEXACT) accq = mfma(lds_slots(Qls, LDK, 16 * ct + n, s, g4), Sh[s], accq);
        }
      }
      Y[ct] = acc;
      OQ[ct] = accq;
    }

    // ---- Z = V - gamma nk Y (beta is in T), as split B operands over c ----
    bf16x8 Zh[2], Zl[2];
    {
      floatx4 Z[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int c = 16 * ct + 4 * g4;
        const uint2 vw = lds_tr4(Vhs + w * VBLK, LDV, c, 0, n);    // V[c + j][rw + n]
        float vv[4] = {bf16lo(vw.x), bf16hi(vw.x), bf16lo(vw.y), bf16hi(vw.y)};
        if constexpr (!KEXACT) {
          const uint2 vl = lds_tr4(Vls + w * VBLK, LDV, c, 0, n);
          vv[0] += bf16lo(vl.x);
          vv[1] += bf16hi(vl.x);
          vv[2] += bf16lo(vl.y);
          vv[3] += bf16hi(vl.y);
        }
        const float4 gg = *reinterpret_cast<const float4*>(&Gs[2 * C + c]);   // gamma nk
        Z[ct] = floatx4{vv[0] - gg.x * Y[ct][0], vv[1] - gg.y * Y[ct][1],
                        vv[2] - gg.z * Y[ct][2], vv[3] - gg.w * Y[ct][3]};
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) split8(acc_slots(Z[2 * s], Z[2 * s + 1]), Zh[s], Zl[s]);
    }

    // ---- U = T diag(beta) Z  (lower triangular: c-tile ct needs k-blocks <= ct/2) ----
    floatx4 U[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= ct / 2; ++s) {
        const bf16x8 th = lds_slots(Ths, LDT, 16 * ct + n, s, g4);
        const bf16x8 tl = lds_slots(Tls, LDT, 16 * ct + n, s, g4);
        acc = mfma(th, Zh[s], acc);
        acc = mfma(th, Zl[s], acc);
        acc = mfma(tl, Zh[s], acc);
      }
      U[ct] = acc;
    }
    bf16x8 Uh[2], Ul[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) split8(acc_slots(U[2 * s], U[2 * s + 1]), Uh[s], Ul[s]);

    // ---- O = diag(gamma) Q S^T + P U ----
#pragma unroll
    for (int ct = 0; ct < 4 && !SC; ++ct) {
      floatx4 acc = OQ[ct];
      const int c = 16 * ct + 4 * g4;
      const float4 gg = *reinterpret_cast<const float4*>(&Gs[c]);          // gamma nq
      acc[0] *= gg.x;
      acc[1] *= gg.y;
      acc[2] *= gg.z;
      acc[3] *= gg.w;
#pragma unroll
      for (int s = 0; s <= ct / 2; ++s) {
        const bf16x8 ph = lds_slots(Phs, LDT, 16 * ct + n, s, g4);
        acc = mfma(ph, Uh[s], acc);
        if constexpr (OPREC) {
          acc = mfma(ph, Ul[s], acc);
          acc = mfma(lds_slots(Pls, LDT, 16 * ct + n, s, g4), Uh[s], acc);
        }
      }
      if constexpr (OPREC) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < nvalid) obase[(size_t)(t0 + c + e) * ostride + n] = acc[e];
      } else {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (bf16)acc[e];
        *reinterpret_cast<bf16x4*>(&Vhs[w * VBLK + n * LDO + c]) = ob;   // O^T[r][c]
      }
    }
    if constexpr (!OPREC && !SC) {
      // O^T of this wave -> 16-byte stores: lane takes token
      // c = 32 m + 16 (g4 >> 1) + n and rows 8 (g4 & 1) .. + 7.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const bf16* Ow = &Vhs[w * VBLK];
      const int rr = 8 * (g4 & 1);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int c0 = 32 * m + 16 * (g4 >> 1);
        const uint2 lo = lds_tr4(Ow, LDO, rr, c0, n);
        const uint2 hi = lds_tr4(Ow, LDO, rr + 4, c0, n);
        if (c0 + n < nvalid)
          *reinterpret_cast<uint4*>(obase + (size_t)(t0 + c0 + n) * ostride + rr) =
              make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }

    // ---- S^T <- gamma_C S^T + K^T diag(e^{g_C - g}) U ----
    {
      bf16x8 Dh[2], Dl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float4 d0 = *reinterpret_cast<const float4*>(&Gs[3 * C + kslot_base(s, g4, 0)]);
        const float4 d1 = *reinterpret_cast<const float4*>(&Gs[3 * C + kslot_base(s, g4, 1)]);
        const floatx4& ua = U[2 * s];
        const floatx4& ub = U[2 * s + 1];
        const floatx8 du = {ua[0] * d0.x, ua[1] * d0.y, ua[2] * d0.z, ua[3] * d0.w,
                            ub[0] * d1.x, ub[1] * d1.y, ub[2] * d1.z, ub[3] * d1.w};
        split8(du, Dh[s], Dl[s]);
      }
      const float gC = Gs[C];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        floatx4 acc = S[dt] * gC;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 kth = lds_slots_tr(Khs, LDK, 16 * dt, s, g4, n);   // K[kslot][16 dt + n]
          acc = mfma(kth, Dh[s], acc);
          acc = mfma(kth, Dl[s], acc);
          if constexpr (!KEXACT) acc = mfma(lds_slots_tr(Kls, LDK, 16 * dt, s, g4, n), Dh[s], acc);
        }
        S[dt] = acc;
      }
    }
  }

  if (ST != nullptr) {
    const size_t srow = (size_t)bh * DV + r0 + rw + n;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<float4*>(ST + srow * DK + 16 * dt + 4 * g4) =
          make_float4(S[dt][0], S[dt][1], S[dt][2], S[dt][3]);
  }
}

// ===========================================================================
// scan, segmented bf16 path: one workgroup per (batch, head, segment)
// ===========================================================================

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_cvoid_t;
// 16 bytes per lane from global memory straight into LDS: lane L's bytes go
// to lds_block + 16 L (lds_block is the same for the whole wave).
__device__ __forceinline__ void dma16(const void* g, void* lds_block) {
  __builtin_amdgcn_global_load_lds((glb_cvoid_t*)g, (lds_void_t*)lds_block, 16, 0, 0);
}

// Index, within one part (hi or lo) of a segment's X^T, at which the scan
// stores element (d, e) (row d of X^T is column d of X; e is the
// contraction index of the combine).  The combine's wave w = d / 16 feeds
// the MFMA, for k-block kb = e / 32, lane (n = d % 16, g4) the 8 k-slots
// e = 32 kb + 4 g4 + i and 32 kb + 16 + 4 g4 + i (i = 0..3); those are
// stored as 16 contiguous bytes, and the 64 lanes' operands for one
// (w, kb) as one contiguous kilobyte, so every operand load reads whole
// cache lines.
// Workgroup execution barrier without a memory fence: orders this wave's
// memory accesses in the compiler only.  Data handed over through it must
// already be complete (here: an explicit wait on the loads that fill LDS),
// and nothing before it waits on this wave's outstanding memory operations.
__device__ __forceinline__ void exec_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int DK>
__device__ __forceinline__ int xfin_index(int d, int e) {
  return ((d >> 4) * (DK / 32) + (e >> 5)) * 512 + (d & 15) * 32 + ((e >> 2) & 3) * 8 +
         ((e >> 4) & 1) * 4 + (e & 3);
}

// The rows a segment evolves are the DV state rows and, for segments >= 1,
// the DK transition rows (see SegArgs).  One workgroup carries all of them:
// wave w owns rows 16 NH w .. 16 NH (w + 1) - 1 of that combined row space
// as NH 16-row slices.  The chunk's K, Q, T, P, V and gate tiles are loaded
// once per workgroup, straight from global memory into one of two LDS
// buffers (direct loads: each wave instruction fills 1 KB, 16 bytes per
// lane) while the previous chunk computes from the other; every operand a
// wave reads from LDS (K, Q, T, P, K^T) serves all NH of its slices.  The
// outputs are formed transposed, O^T = S Q^T diag(gamma) + U^T P^T, so a
// lane holds 4 consecutive rows of one token and stores them directly.
// Segment 0 has no transition rows; its transition waves only load tiles.
template <int DK, int DV, int NH>
__global__ __launch_bounds__(64 * (DV + DK) / (16 * NH), 1) void scan_wide_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k,
    const bf16* __restrict__ v, const float* S0, bf16* __restrict__ o,
    const float* __restrict__ ws, int T, int H, int nchunks, SegArgs seg) {
  constexpr int RPW = 16 * NH;          // rows per wave
  static_assert(DV % RPW == 0 && DK % RPW == 0, "waves hold state or transition rows only");
  constexpr int NW = (DV + DK) / RPW;   // waves
  constexpr int NDT = DK / 16;          // d-tiles of a 16-row state slice
  constexpr int NKB = DK / 32;          // 32-wide k-blocks over d
  // Tiles are row-major bf16 with one 16-byte pad unit per row (strides of
  // an odd number of 16-byte units keep row-parallel reads on distinct
  // banks).  UK, UT, UV: 16-byte units per row including the pad.
  constexpr int LDK = DK + 8, LDT = C + 8, LDV = DV + 8;
  constexpr int UK = LDK / 8, UT = LDT / 8, UV = LDV / 8;
  // one buffer: K, Q [C][LDK]; T hi, T lo, P [C][LDT]; V [C][LDV]; gates fp32
  // [4][C]; the exponent rows of P fp32 [2][C] (in a 1 KB load block).  P is
  // formed here from K and Q; everything else is loaded.
  constexpr int OFF_Q = C * LDK, OFF_T = 2 * C * LDK, OFF_V = OFF_T + 3 * C * LDT;
  constexpr int OFF_P = OFF_T + 2 * C * LDT;
  constexpr int OFF_G = OFF_V + C * LDV;
  constexpr int OFF_AB = OFF_G + 2 * 4 * C;
  constexpr int BUF = OFF_AB + 512;                      // bf16 elements
  // 1 KB load blocks per buffer (64 rows of U units = U blocks per tile)
  constexpr int NBK = UK, NBT = 2 * UT, NBV = UV;
  __shared__ __attribute__((aligned(16))) bf16 buf0[BUF];
  __shared__ __attribute__((aligned(16))) bf16 buf1[BUF];

  const int bh = blockIdx.x / seg.nseg, sg = blockIdx.x - bh * seg.nseg;
  const int b = bh / H, h = bh - b * H;
  const int c_begin = sg * seg.seg_chunks;
  const int c_end = min(c_begin + seg.seg_chunks, nchunks);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int n = lane & 15, g4 = lane >> 4;
  const int row0 = RPW * w;                 // first row (combined space)
  const bool xrows = row0 >= DV;            // transition rows
  const bool active = !xrows || sg > 0;

  const bf16* k_seq = k + ((size_t)b * T * H + h) * DK;
  const bf16* q_seq = q + ((size_t)b * T * H + h) * DK;
  const bf16* v_seq = v + ((size_t)b * T * H + h) * DV;
  const size_t tok_k = (size_t)H * DK, tok_v = (size_t)H * DV;

  // Issue this wave's share of the load blocks of `chunk` into buffer X.
  // Every wave takes the same number of blocks of each tile (block
  // w + NW j): their types are known at compile time, the code is
  // branch-free, and K, Q (and V, when its rows have the same length) share
  // one row/unit computation.  The few blocks left over, and the gate block,
  // go one per wave.  A lane whose 16 bytes land on a pad unit fetches the
  // row's first unit (never read).  Token rows past the end of the sequence
  // load the last valid row: their beta is 0 and their decay 1, so they
  // contribute nothing (finite values times zero) and their outputs are not
  // stored.
  constexpr int MK = NBK / NW, MT = NBT / NW, MV = NBV / NW;   // blocks per wave
  constexpr int EK = NBK - NW * MK, ET = NBT - NW * MT, EV = NBV - NW * MV;
  constexpr int NE = 2 * EK + ET + EV + 2;                      // left over
  auto issue = [&](bf16* X, int chunk) {
    const int t0 = chunk * C;
    const int last = min(C, T - t0) - 1;
    const char* wsc = reinterpret_cast<const char*>(ws) +
                      ((size_t)bh * nchunks + chunk) * kChunkWsFloats * 4;
    const bf16* kc = k_seq + (size_t)t0 * tok_k;
    const bf16* qc = q_seq + (size_t)t0 * tok_k;
    const bf16* vc = v_seq + (size_t)t0 * tok_v;
    // The per-lane offsets below do not depend on the chunk; an opaque copy
    // of the lane index keeps the compiler from hoisting them out of the
    // chunk loop, where they would take registers the compute needs.
    unsigned ln = lane;
    asm volatile("" : "+v"(ln));
    const unsigned lastu = last;
    // element offset, from the chunk's first row, of lane's unit in block jb
    // of a tile with U units per row and a row stride of tok elements
    auto row_off = [&](unsigned jb, unsigned U, unsigned tok) -> unsigned {
      const unsigned idx = 64 * jb + ln, row = idx / U, u = idx - row * U;
      return min(row, lastu) * tok + 8 * (u < U - 1 ? u : 0);
    };
    // byte offset in the chunk's workspace of lane's unit in block jt of the
    // T hi / T lo / P hi tiles
    auto tp_off = [&](unsigned jt) -> unsigned {
      const unsigned idx = 64 * jt + ln;
      const unsigned m = idx / (C * UT), rm = idx - m * (C * UT);
      const unsigned row = rm / UT, u = rm - row * UT;
      return m * (C * C * 2) + row * (C * 2) + 16 * (u < UT - 1 ? u : 0);
    };
#pragma unroll
    for (int j = 0; j < MK; ++j) {
      const int jb = w + NW * j;
      const unsigned off = row_off(jb, UK, tok_k);
      dma16(kc + off, X + 512 * jb);
      dma16(qc + off, X + OFF_Q + 512 * jb);
      if constexpr (DV == DK) dma16(vc + off, X + OFF_V + 512 * jb);   // same geometry
    }
#pragma unroll
    for (int j = (DV == DK ? MK : 0); j < MV; ++j) {
      const int jb = w + NW * j;
      dma16(vc + row_off(jb, UV, tok_v), X + OFF_V + 512 * jb);
    }
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int jt = w + NW * j;
      dma16(wsc + tp_off(jt), X + OFF_T + 512 * jt);
    }
    for (int e = w; e < NE; e += NW) {
      if (e < 2 * EK) {
        const int jb = NW * MK + (e < EK ? e : e - EK);
        dma16((e < EK ? kc : qc) + row_off(jb, UK, tok_k),
              X + (e < EK ? 0 : OFF_Q) + 512 * jb);
      } else if (e < 2 * EK + ET) {
        const int jt = NW * MT + e - 2 * EK;
        dma16(wsc + tp_off(jt), X + OFF_T + 512 * jt);
      } else if (e < 2 * EK + ET + EV) {
        const int jb = NW * MV + e - 2 * EK - ET;
        dma16(vc + row_off(jb, UV, tok_v), X + OFF_V + 512 * jb);
      } else if (e == 2 * EK + ET + EV) {
        dma16(wsc + kWsG + 16 * ln, X + OFF_G);
      } else {
        dma16(wsc + kWsAB + 16 * ln, X + OFF_AB);
      }
    }
  };
  static_assert(OFF_Q == 512 * NBK && OFF_T == 512 * 2 * NBK && OFF_P == OFF_T + 512 * NBT &&
                OFF_V == OFF_P + 512 * UT && OFF_G == OFF_V + 512 * NBV &&
                OFF_AB == OFF_G + 512, "load blocks and P tile the buffer");

  // P's upper tiles that the scan reads, (0,1) and (2,3), are zero in both
  // buffers for good (no load writes P's space)
  for (int idx = tid; idx < 2 * 256; idx += 64 * NW) {
    const int tl = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
    const int off = OFF_P + (32 * tl + r) * LDT + 32 * tl + 16 + cc;
    buf0[off] = bf16(0.f);
    buf1[off] = bf16(0.f);
  }

  // ---- carried state: S^T tiles of each slice, lane holds
  //      S^T[d = 16 dt + 4 g4 + i][row = 16 hf + n] ----
  floatx4 S[NH][NDT];
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
    const int r = row0 + 16 * hf + n;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (xrows) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[hf][dt][i] = (16 * dt + 4 * g4 + i == r - DV) ? 1.f : 0.f;
      } else if (S0 != nullptr && sg == 0) {
        const float4 x = *reinterpret_cast<const float4*>(
            S0 + ((size_t)bh * DV + r) * DK + 16 * dt + 4 * g4);
        S[hf][dt] = floatx4{x.x, x.y, x.z, x.w};
      } else {
        S[hf][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // Outputs: o for state rows, x^_t = X_t q_t ([BH][T][DK]) for transition
  // rows; obase + t * ostride is token t's element for this wave's row 0.
  bf16* obase;
  size_t ostride;
  if (xrows) {
    obase = reinterpret_cast<bf16*>(seg.xhat) + (size_t)bh * T * DK + (row0 - DV);
    ostride = DK;
  } else {
    obase = o + ((size_t)b * T * H + h) * DV + row0;
    ostride = (size_t)H * DV;
  }

  // One chunk from buffer X (loaded), prefetching chunk + 1 into buffer Nx.
  auto step = [&](bf16* X, bf16* Nx, int chunk) {
    const int t0 = chunk * C;
    const int nvalid = min(C, T - t0);
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this wave's loads of X
    __syncthreads();                          // everyone's loads of X; Nx is free
    if (chunk + 1 < c_end) issue(Nx, chunk + 1);
    const bf16* Ks = X;
    const bf16* Qs = X + OFF_Q;
    const bf16* Ths = X + OFF_T;
    const bf16* Tls = Ths + C * LDT;
    const bf16* Phs = X + OFF_P;
    const bf16* Vs = X + OFF_V;
    const float* Gs = reinterpret_cast<const float*>(X + OFF_G);

    // ---- P_ji = 2^(a_j - b_i) q~_j . k~_i for i <= j: the ten lower 16x16
    //      tiles, shared out over the waves (tile (mi, ni): a lane holds row
    //      j = 16 mi + n, columns 16 ni + 4 g4 .. + 3); read after the
    //      barrier before the outputs ----
    {
      // an opaque copy of the lane index keeps these per-lane addresses from
      // being hoisted out of the chunk loop (registers the products need)
      unsigned ln = lane;
      asm volatile("" : "+v"(ln));
      const int pn = ln & 15, pg = ln >> 4;
      const float* Ab = reinterpret_cast<const float*>(X + OFF_AB);
      for (int tp = w; tp < 10; tp += NW) {
        const int mi = tp >= 6 ? 3 : tp >= 3 ? 2 : tp >= 1 ? 1 : 0;
        const int ni = tp - mi * (mi + 1) / 2;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NKB; ++s)
          acc = mfma(lds_slots(Ks, LDK, 16 * ni + pn, s, pg),
                     lds_slots(Qs, LDK, 16 * mi + pn, s, pg), acc);
        const int j = 16 * mi + pn, i0 = 16 * ni + 4 * pg;
        const float aj = Ab[j];
        const float4 b4 = *reinterpret_cast<const float4*>(&Ab[C + i0]);
        const float bi[4] = {b4.x, b4.y, b4.z, b4.w};
        bf16x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pv[e] = (bf16)(i0 + e <= j ? __builtin_amdgcn_exp2f(aj - bi[e]) * acc[e] : 0.f);
        *reinterpret_cast<bf16x4*>(X + OFF_P + j * LDT + i0) = pv;
      }
    }
    __builtin_amdgcn_sched_barrier(0);        // keep P's registers out of the products below
    if (!active) {
      __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): this wave's P tiles
      exec_barrier();
      return;
    }

    // ---- Y = K S^T for all slices (c-tile ct: rows c = 16 ct + 4 g4 + i,
    //      col = row n of the slice) ----
    floatx4 Y[NH][4];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) Y[hf][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    // the hi parts of the split state are S rounded to bf16: kept for O
    bf16x8 Sh[NKB][NH];
#pragma unroll
    for (int s = 0; s < NKB; ++s) {
      bf16x8 Sl[NH];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
        split8(acc_slots(S[hf][2 * s], S[hf][2 * s + 1]), Sh[s][hf], Sl[hf]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16x8 kh = lds_slots(Ks, LDK, 16 * ct + n, s, g4);
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
          Y[hf][ct] = mfma(kh, Sh[s][hf], Y[hf][ct]);
          Y[hf][ct] = mfma(kh, Sl[hf], Y[hf][ct]);
        }
      }
    }

    // ---- Z = V - gamma nk Y (beta is in T), as split B operands over c ----
    const uint32_t vmask = xrows ? 0u : 0xFFFFFFFFu;
    bf16x8 Zh[NH][2], Zl[NH][2];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      floatx4 Z[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int c = 16 * ct + 4 * g4;
        // V[c + j][row]; transition rows read column 0 and mask it to 0
        // (branch-free, so the read stays in the block the load tracking
        // knows does not touch the buffer being filled)
        const uint2 vr = lds_tr4(Vs, LDV, c, xrows ? 0 : row0 + 16 * hf, n);
        const uint2 vw = make_uint2(vr.x & vmask, vr.y & vmask);
        const float vv[4] = {bf16lo(vw.x), bf16hi(vw.x), bf16lo(vw.y), bf16hi(vw.y)};
        const float4 gg = *reinterpret_cast<const float4*>(&Gs[2 * C + c]);   // gamma nk
        Z[ct] = floatx4{vv[0] - gg.x * Y[hf][ct][0], vv[1] - gg.y * Y[hf][ct][1],
                        vv[2] - gg.z * Y[hf][ct][2], vv[3] - gg.w * Y[hf][ct][3]};
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) split8(acc_slots(Z[2 * s], Z[2 * s + 1]), Zh[hf][s], Zl[hf][s]);
    }

    // ---- U = T diag(beta) Z  (lower triangular: c-tile ct needs k-blocks <= ct/2) ----
    floatx4 U[NH][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) U[hf][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= ct / 2; ++s) {
        const bf16x8 th = lds_slots(Ths, LDT, 16 * ct + n, s, g4);
        const bf16x8 tl = lds_slots(Tls, LDT, 16 * ct + n, s, g4);
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
          U[hf][ct] = mfma(th, Zh[hf][s], U[hf][ct]);
          U[hf][ct] = mfma(th, Zl[hf][s], U[hf][ct]);
          U[hf][ct] = mfma(tl, Zh[hf][s], U[hf][ct]);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): this wave's P tiles
    exec_barrier();                           // every wave's P tiles are in LDS

    // ---- O^T = S Q^T diag(gamma) + U^T P^T (single-pass bf16: o is bf16);
    //      tile ct: rows r = 4 g4 + i of the slice, token c = 16 ct + n ----
    {
      floatx4 OT[NH][4];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) OT[hf][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKB; ++s) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const bf16x8 qh = lds_slots(Qs, LDK, 16 * ct + n, s, g4);
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) OT[hf][ct] = mfma(Sh[s][hf], qh, OT[hf][ct]);
        }
      }
      bf16x8 Uh[NH][2];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
#pragma unroll
        for (int s = 0; s < 2; ++s) Uh[hf][s] = to_bf16x8(acc_slots(U[hf][2 * s], U[hf][2 * s + 1]));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const float gam = Gs[16 * ct + n];                                 // gamma nq
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) OT[hf][ct] *= gam;
#pragma unroll
        for (int s = 0; s <= ct / 2; ++s) {
          const bf16x8 ph = lds_slots(Phs, LDT, 16 * ct + n, s, g4);
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) OT[hf][ct] = mfma(Uh[hf][s], ph, OT[hf][ct]);
        }
        const int c = 16 * ct + n;
        if (c < nvalid) {
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) {
            bf16x4 ob;
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[e] = (bf16)OT[hf][ct][e];
            *reinterpret_cast<bf16x4*>(obase + (size_t)(t0 + c) * ostride + 16 * hf + 4 * g4) = ob;
          }
        }
      }
    }

    // ---- S^T <- gamma_C S^T + K^T diag(e^{g_C - g}) U, all slices ----
    {
      bf16x8 Dh[NH][2], Dl[NH][2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float4 d0 = *reinterpret_cast<const float4*>(&Gs[3 * C + kslot_base(s, g4, 0)]);
        const float4 d1 = *reinterpret_cast<const float4*>(&Gs[3 * C + kslot_base(s, g4, 1)]);
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
          const floatx4& ua = U[hf][2 * s];
          const floatx4& ub = U[hf][2 * s + 1];
          const floatx8 du = {ua[0] * d0.x, ua[1] * d0.y, ua[2] * d0.z, ua[3] * d0.w,
                              ub[0] * d1.x, ub[1] * d1.y, ub[2] * d1.z, ub[3] * d1.w};
          split8(du, Dh[hf][s], Dl[hf][s]);
        }
      }
      const float gC = Gs[C];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S[hf][dt] *= gC;
      // k-block outer: the NH * NDT state tiles are independent MFMA chains
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 kth = lds_slots_tr(Ks, LDK, 16 * dt, s, g4, n);   // K[kslot][16 dt + n]
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) {
            S[hf][dt] = mfma(kth, Dh[hf][s], S[hf][dt]);
            S[hf][dt] = mfma(kth, Dl[hf][s], S[hf][dt]);
          }
        }
      }
    }
  };

  issue(buf0, c_begin);
  for (int chunk = c_begin; chunk < c_end; chunk += 2) {
    step(buf0, buf1, chunk);
    if (chunk + 1 < c_end) step(buf1, buf0, chunk + 1);
  }

  // Final rows of this segment for the combine pass: state rows as fp32,
  // transition rows as X^T split into bf16 hi and lo parts, in the order
  // xfin_index gives (the combine loads them as MFMA operands).
  if (active && !xrows) {
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      float* dst = seg.S_fin + (((size_t)bh * seg.nseg + sg) * DV + row0 + 16 * hf + n) * DK;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<float4*>(dst + 16 * dt + 4 * g4) =
            make_float4(S[hf][dt][0], S[hf][dt][1], S[hf][dt][2], S[hf][dt][3]);
    }
  } else if (active) {
    bf16* xh = reinterpret_cast<bf16*>(seg.X_fin) + ((size_t)bh * seg.nseg + sg) * 2 * DK * DK;
    bf16* xl = xh + DK * DK;
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const int e = row0 - DV + 16 * hf + n;             // row of X
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * dt + 4 * g4 + i;            // column of X
          bf16 hi, lo;
          split_bf16(S[hf][dt][i], hi, lo);
          xh[xfin_index<DK>(d, e)] = hi;
          xl[xfin_index<DK>(d, e)] = lo;
        }
    }
  }
}

// ===========================================================================
// T == 0: the final state is the initial one (or zero)
// ===========================================================================

__global__ void state_fill_kernel(const float* S0, float* ST, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ST[i] = S0 ? S0[i] : 0.f;
}

hipError_t launch_state_fill(const float* S0, float* ST, size_t n,
                             hipStream_t stream) {
  if (n == 0 || ST == nullptr || ST == S0) return hipSuccess;
  hipLaunchKernelGGL(state_fill_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, S0, ST, n);
  return hipGetLastError();
}

// ===========================================================================
// launchers
// ===========================================================================

template <int DK, typename TIn, bool GATHER>
static void launch_prepare_t(const void* q, const void* k, const float* alpha,
                             const float* beta, float* ws, int B, int T, int H,
                             bool write_pl, bool scan_forms_p, const QkArgs& qa,
                             hipStream_t stream) {
  const int nchunks = (T + C - 1) / C;
  if constexpr (std::is_same<TIn, bf16>::value) {
    if (scan_forms_p) {
      hipLaunchKernelGGL((prepare_kernel<DK, TIn, GATHER, true>), dim3(nchunks, H, B),
                         dim3(64), 0, stream, static_cast<const TIn*>(q),
                         static_cast<const TIn*>(k), alpha, beta, ws, T, H, nchunks, 0, qa);
      return;
    }
  }
  hipLaunchKernelGGL((prepare_kernel<DK, TIn, GATHER, false>), dim3(nchunks, H, B), dim3(64),
                     0, stream, static_cast<const TIn*>(q),
                     static_cast<const TIn*>(k), alpha, beta, ws, T, H,
                     nchunks, write_pl ? 1 : 0, qa);
}

hipError_t launch_prefill_prepare(const void* q, const void* k,
                                  const float* alpha, const float* beta,
                                  float* ws, int B, int T, int H, int dk,
                                  int in_dtype, bool write_pl, bool scan_forms_p,
                                  const QkArgs& qa, hipStream_t stream) {
#define GDN_PREP(DK, TI, G) \
  launch_prepare_t<DK, TI, G>(q, k, alpha, beta, ws, B, T, H, write_pl, scan_forms_p, qa, stream)
  const bool g = qa.chan != nullptr;
  if (in_dtype == 1) {
    if (dk == 128) { if (g) GDN_PREP(128, bf16, true); else GDN_PREP(128, bf16, false); }
    else { if (g) GDN_PREP(64, bf16, true); else GDN_PREP(64, bf16, false); }
  } else {
    if (dk == 128) { if (g) GDN_PREP(128, float, true); else GDN_PREP(128, float, false); }
    else { if (g) GDN_PREP(64, float, true); else GDN_PREP(64, float, false); }
  }
#undef GDN_PREP
  return hipGetLastError();
}

// ===========================================================================
// segment combine (phase 2): S_in(s) = S_end(s-1), S_end(s) = S_in(s) X_s + S_loc(s)
// ===========================================================================

// One workgroup per (batch, head, 16 state rows), sequential over the
// segments.  DK / 16 compute waves; wave w forms columns 16 w .. 16 w + 15
// of S_end(s) = S_in(s) X_s + S_loc(s) for the 16 rows with three short
// MFMA chains (hi x hi, hi x lo, lo x hi).  Its operand rows of X_s^T
// (8 KB) and its S_loc tile come straight from global memory into
// registers two segments ahead (a ring of three register sets, the loop
// unrolled by three so every index is static), so the loads' latency is
// hidden behind two steps.  The waves exchange the hi/lo split of S_in(s)
// through a double-buffered LDS tile, one fence-free barrier per segment.
// Compute waves issue no store inside the loop (their partial load waits
// stay exact); a copier wave writes the hi part of S_in(s), i.e. S_in(s)
// rounded to bf16, out for the correction pass.
template <int DK>
__global__ __launch_bounds__(64 * (DK / 16 + 1)) void segment_combine_kernel(
    SegArgs seg, float* ST, int DV) {
  constexpr int NWC = DK / 16;
  constexpr int NKB = DK / 32;
  constexpr int LDE = DK + 8;                   // padded row of the exchanged S_in split
  constexpr int ET = 16 * LDE;                  // elements of one part of it
  constexpr int NBS = 16 * DK * 2 / 1024;       // 1 KB blocks of the 16 rows' bf16 S_in
  __shared__ __attribute__((aligned(16))) bf16 sx[2][2 * ET];
  // Consecutive workgroups go to different XCDs (each with its own L2).
  // Workgroup i takes head i % BH: when BH is a multiple of the XCD count,
  // the row groups of one head share an XCD, and its L2 serves their
  // common reads of X.
  const int BH = gridDim.x / (DV / 16);
  const int bh = blockIdx.x % BH, rg = blockIdx.x / BH;
  const int r0 = 16 * rg;                       // first state row of the workgroup
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const int nseg = seg.nseg;

  // Steps run in groups of three (the compute loop is unrolled by three so
  // that no load sits in a conditional branch, which would make the
  // compiler's load-count waits drain everything); steps past the last
  // segment pass the barrier and publish nothing.
  const int nsteps = 3 * ((nseg - 1 + 2) / 3);

  if (w == NWC) {
    // ---------------- copier ----------------
    for (int s = 1; s <= nsteps; ++s) {
      exec_barrier();                           // the split of S_in(s) is in LDS
      if (s >= nseg) continue;
#pragma unroll
      for (int j = 0; j < NBS; ++j) {
        const int idx = 64 * j + lane, row = idx / (DK / 8), u = idx - row * (DK / 8);
        const uint4 x = *reinterpret_cast<const uint4*>(&sx[s & 1][row * LDE + 8 * u]);
        bf16* dst = reinterpret_cast<bf16*>(seg.S_in) +
                    (((size_t)bh * nseg + s) * DV + r0 + row) * DK + 8 * u;
        *reinterpret_cast<uint4*>(dst) = x;
      }
    }
    return;
  }

  // ---------------- compute ----------------
  // lane holds S[r0 + n][16 w + 4 g4 + i], i = 0..3 (an S^T accumulator tile)
  auto tile = [&](int s) {
    const float4 x = *reinterpret_cast<const float4*>(
        seg.S_fin + (((size_t)bh * nseg + s) * DV + r0 + n) * DK + 16 * w + 4 * g4);
    return floatx4{x.x, x.y, x.z, x.w};
  };
  // X_s^T row 16 w + n, k-slots of lane group g4 (xfin_index: k-block kb
  // is 512 elements further): hi parts [0, NKB), lo parts [NKB, 2 NKB), and
  // S_loc(s).  Segments past the end load the last
  // one (never used), so the loads are unconditional.
  auto load = [&](bf16x8* X, floatx4& L, int s) {
    s = min(s, nseg - 1);
    const bf16* src = reinterpret_cast<const bf16*>(seg.X_fin) +
                      ((size_t)bh * nseg + s) * 2 * DK * DK + xfin_index<DK>(16 * w + n, 4 * g4);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      X[kb] = *reinterpret_cast<const bf16x8*>(src + 512 * kb);
      X[NKB + kb] = *reinterpret_cast<const bf16x8*>(src + DK * DK + 512 * kb);
    }
    L = tile(s);
  };
  // hi/lo split of this lane's 4 values into exchange buffer e
  auto publish = [&](const floatx4& v, int e) {
    const float x[4] = {v[0], v[1], v[2], v[3]};
    bf16x4 hi, lo;
    split4(x, hi, lo);
    *reinterpret_cast<bf16x4*>(&sx[e][n * LDE + 16 * w + 4 * g4]) = hi;
    *reinterpret_cast<bf16x4*>(&sx[e][ET + n * LDE + 16 * w + 4 * g4]) = lo;
  };
  floatx4 S, Sfinal;
  // segment s with operands X, L; reloads the set for segment s + 2 into Xn, Ln
  auto step = [&](int s, const bf16x8* X, const floatx4& L, bf16x8* Xn, floatx4& Ln) {
    __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): this wave's split is in LDS
    exec_barrier();                             // everyone's split of S_in(s) visible
    const bf16* E = sx[s & 1];
    // all operand reads first (one LDS latency), and the loads for segment
    // s + 2 before the products, so the address units drain them meanwhile
    bf16x8 bh8[NKB], bl8[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      bh8[kb] = lds_slots(E, LDE, n, kb, g4);         // S_in(s)[r0 + n][e], hi
      bl8[kb] = lds_slots(E + ET, LDE, n, kb, g4);    // lo
    }
    load(Xn, Ln, s + 2);
    __builtin_amdgcn_sched_barrier(0);
    floatx4 a0 = L, a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      a0 = mfma(X[kb], bh8[kb], a0);
      a1 = mfma(X[kb], bl8[kb], a1);
      a2 = mfma(X[NKB + kb], bh8[kb], a2);
    }
    S = a0 + (a1 + a2);                         // S_end(s)
    const bool last = s == nseg - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) Sfinal[i] = last ? S[i] : Sfinal[i];
    if (s + 1 < nseg) publish(S, (s + 1) & 1);
  };
  bf16x8 XA[2 * NKB], XB[2 * NKB], XC[2 * NKB];
  floatx4 LA, LB, LC;
  S = tile(0);                                  // S_end(0), the first load waited on
  load(XA, LA, 1);
  load(XB, LB, 2);
  publish(S, 1);
  for (int s = 1; s <= nsteps; s += 3) {
    step(s, XA, LA, XC, LC);
    step(s + 1, XB, LB, XA, LA);
    step(s + 2, XC, LC, XB, LB);
  }
  if (ST != nullptr)
    *reinterpret_cast<float4*>(ST + ((size_t)bh * DV + r0 + n) * DK + 16 * w + 4 * g4) =
        make_float4(Sfinal[0], Sfinal[1], Sfinal[2], Sfinal[3]);
}

// ===========================================================================
// segment correction (phase 3): o_t += S_in(s) x^_t for tokens of segments >= 1
// ===========================================================================

// One workgroup per (batch, head, segment >= 1), in two roles:
//  * two loader waves, one for the segment's x^ tiles and one for its (old)
//    o tiles, move them 64 tokens at a time straight from global memory into
//    a ring of three LDS buffers, two tiles ahead.  They issue nothing but
//    these loads, so waiting for the oldest tile is an exact partial wait on
//    their own load counter.  (Issuing a tile takes as long as the memory
//    system accepts it: the pass runs at about 4.3 TB/s, and a deeper ring
//    or cheaper address arithmetic measured no faster.)
//  * DV/16 compute waves (wave w: state rows 16 w .. 16 w + 15) form
//    O_corr^T = S_in x^^T for each tile (S_in as the resident A operand; a
//    lane holds 4 consecutive rows of one token), add the old o from LDS and
//    store.  They never wait on memory: with stores in flight, a wave's load
//    counter could only be waited down to zero.
// The roles run separate loops (the branch is uniform per wave) that pass
// the same barriers, one per tile.  Single-pass bf16 (outputs are bf16).
constexpr int kCorrLoaders = 2;

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 16 + kCorrLoaders)) void segment_correct_kernel(
    SegArgs seg, bf16* o, int T, int H) {
  constexpr int NKB = DK / 32;
  constexpr int NCW = DV / 16;                   // compute waves
  constexpr int LDXH = DK + 8, UXH = LDXH / 8;   // padded x^ tile row (16-byte units)
  constexpr int LDOT = DV + 8, UOT = LDOT / 8;   // padded o tile row
  constexpr int XT = C * LDXH, OT = C * LDOT;    // elements per tile
  static_assert(kCorrLoaders == 2, "one loader wave per tile");
  static_assert(UXH <= 63 && UOT <= 63, "one tile's loads fit the load counter");
  constexpr int NBUF = 3;
  __shared__ __attribute__((aligned(16))) bf16 ring[NBUF][XT + OT];

  const int nsl = seg.nseg - 1;
  const int bh = blockIdx.x / nsl, s = 1 + (blockIdx.x - (blockIdx.x / nsl) * nsl);
  const int b = bh / H, h = bh - b * H;
  const int t_begin = s * seg.seg_chunks * C;
  const int t_end = min(T, t_begin + seg.seg_chunks * C);
  const int ngroups = (t_end - t_begin + C - 1) / C;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g4 = lane >> 4;
  const bf16* xh = reinterpret_cast<const bf16*>(seg.xhat) + (size_t)bh * T * DK;
  bf16* ob = o + ((size_t)b * T * H + h) * DV;   // + t * H * DV
  const size_t tok_o = (size_t)H * DV;

  if (w >= NCW) {
    // ---------------- loaders: the first x^ tiles, the second o tiles ----
    // A tile of 64 rows of U 16-byte units (one of them padding) is U blocks
    // of 1 KB.  Each lane's offset in every block, from the tile's first
    // row, is computed once; a tile then costs a scalar base and one add per
    // block.  Rows past the sequence end (its last, partial tile only) load
    // the last row instead and are never stored.
    auto run = [&](auto u_c, const bf16* src, int stride, int dst_off) {
      constexpr int U = decltype(u_c)::value;
      int off[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int idx = 64 * j + lane, row = idx / U, u = idx - row * U;
        off[j] = row * stride + 8 * (u < U - 1 ? u : 0);   // pad units: unit 0
      }
      auto issue = [&](int g) {
        bf16* buf = ring[g % NBUF] + dst_off;
        const int t0 = t_begin + C * g;
        const bf16* base = src + (size_t)t0 * stride;
        if (t0 + C <= t_end) {
#pragma unroll
          for (int j = 0; j < U; ++j) dma16(base + off[j], buf + 512 * j);
        } else {
#pragma unroll
          for (int j = 0; j < U; ++j) {
            const int idx = 64 * j + lane, row = idx / U, u = idx - row * U;
            dma16(base + min(row, t_end - 1 - t0) * stride + 8 * (u < U - 1 ? u : 0),
                  buf + 512 * j);
          }
        }
      };
      issue(0);
      if (ngroups > 1) issue(1);
      for (int g = 0; g < ngroups; ++g) {
        // tile g complete (tile g + 1 may still be in flight)
        if (g + 1 < ngroups)
          __builtin_amdgcn_s_waitcnt(0x0F70 | (U & 15) | ((U >> 4) << 14));
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);
        exec_barrier();                // tile g visible; tile g - 1's buffer is free
        if (g + 2 < ngroups) issue(g + 2);
      }
    };
    if (w == NCW)
      run(std::integral_constant<int, UXH>{}, xh, DK, 0);
    else
      run(std::integral_constant<int, UOT>{}, ob, (int)tok_o, XT);
    return;
  }

  // ---------------- compute ----------------
  const int r0 = 16 * w;                         // first row of this wave
  const bf16* sin_row = reinterpret_cast<const bf16*>(seg.S_in) +
                        (((size_t)bh * seg.nseg + s) * DV + r0 + n) * DK;
  bf16x8 As[NKB];                                // A operand: S_in[r0 + n][32 kb + 8 g4 .. + 7]
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    As[kb] = *reinterpret_cast<const bf16x8*>(sin_row + 32 * kb + 8 * g4);
  for (int g = 0; g < ngroups; ++g) {
    exec_barrier();                    // tile g loaded
    const bf16* xs = ring[g % NBUF];
    const bf16* os = xs + XT;
    const int t0 = t_begin + C * g;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int c = 16 * tt + n;                 // token of this lane
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)   // k-slots d = 32 kb + 8 g4 .. + 7, as in As
        acc = mfma(As[kb], *reinterpret_cast<const bf16x8*>(&xs[c * LDXH + 32 * kb + 8 * g4]), acc);
      // acc[i] = O_corr[token c][row r0 + 4 g4 + i]
      const bf16x4 old = *reinterpret_cast<const bf16x4*>(&os[c * LDOT + r0 + 4 * g4]);
      bf16x4 nv;
#pragma unroll
      for (int i = 0; i < 4; ++i) nv[i] = (bf16)((float)old[i] + acc[i]);
      if (t0 + c < t_end)
        *reinterpret_cast<bf16x4*>(ob + (size_t)(t0 + c) * tok_o + r0 + 4 * g4) = nv;
    }
  }
}

// ===========================================================================
// scan launcher
// ===========================================================================

// Waves per scan_kernel workgroup (16 state rows each).
constexpr int kScanWaves = 4;

// 16-row slices per wave of scan_wide_kernel.
constexpr int kWideSlices = 2;

// CUs of the target GPU (MI355X); grids larger than this use the
// two-workgroups-per-CU build of the bf16 scan.
constexpr int kNumCUs = 256;

// Unsegmented scans run scan_kernel (one workgroup per head and 64 state
// rows); segmented ones (bf16 in and out only) run scan_wide_kernel, one
// workgroup per head and segment.
template <int DK, typename TIn, typename TOut>
static void launch_scan_t(const void* q, const void* k, const void* v,
                          const float* S0, void* o, float* ST, const float* ws,
                          int B, int T, int H, int dv, const SegArgs& seg,
                          hipStream_t stream) {
  const int nchunks = (T + C - 1) / C;
  constexpr bool BF16IO = std::is_same<TIn, bf16>::value && std::is_same<TOut, bf16>::value;
  if constexpr (BF16IO) {
    if (seg.nseg > 1) {
#define GDN_WIDE(DV_)                                                               \
  hipLaunchKernelGGL((scan_wide_kernel<DK, DV_, kWideSlices>), dim3(B * H * seg.nseg), \
                     dim3(64 * (DV_ + DK) / (16 * kWideSlices)), 0, stream,         \
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k),      \
                     static_cast<const bf16*>(v), S0, static_cast<bf16*>(o), ws, T, \
                     H, nchunks, seg)
      if (dv == 128) GDN_WIDE(128);
      else GDN_WIDE(64);
#undef GDN_WIDE
      return;
    }
  }
  constexpr int ROWS = 16 * kScanWaves;
  const int nblocks = B * H * (dv / ROWS);
  if (BF16IO && nblocks > kNumCUs) {
    hipLaunchKernelGGL((scan_kernel<DK, TIn, TOut, kScanWaves, 2>), dim3(nblocks),
                       dim3(64 * kScanWaves), 0, stream,
                       static_cast<const TIn*>(q), static_cast<const TIn*>(k),
                       static_cast<const TIn*>(v), S0, static_cast<TOut*>(o), ST,
                       ws, T, H, dv, nchunks, nblocks, nullptr);
  } else {
    hipLaunchKernelGGL((scan_kernel<DK, TIn, TOut, kScanWaves, 1>), dim3(nblocks),
                       dim3(64 * kScanWaves), 0, stream,
                       static_cast<const TIn*>(q), static_cast<const TIn*>(k),
                       static_cast<const TIn*>(v), S0, static_cast<TOut*>(o), ST,
                       ws, T, H, dv, nchunks, nblocks, nullptr);
  }
}

// The backward pass's forward sweep (bf16 inputs): the state at the start of
// every chunk into Sc, no outputs.  ws holds the prepare phase's tiles.
hipError_t launch_scan_states(const void* k, const void* v, const float* S0,
                              const float* ws, float* Sc, int B, int T, int H,
                              int dk, int dv, hipStream_t stream) {
  const int nchunks = (T + C - 1) / C;
  constexpr int ROWS = 16 * kScanWaves;
  const int nblocks = B * H * (dv / ROWS < 1 ? 1 : dv / ROWS);
#define GDN_SC(DK_, MW)                                                                    \
  hipLaunchKernelGGL((scan_kernel<DK_, bf16, bf16, kScanWaves, MW, true>), dim3(nblocks), \
                     dim3(64 * kScanWaves), 0, stream, static_cast<const bf16*>(k),        \
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v), S0,         \
                     static_cast<bf16*>(nullptr), static_cast<float*>(nullptr), ws, T, H,  \
                     dv, nchunks, nblocks, Sc)
  if (dk == 128) { if (nblocks > kNumCUs) GDN_SC(128, 2); else GDN_SC(128, 1); }
  else { if (nblocks > kNumCUs) GDN_SC(64, 2); else GDN_SC(64, 1); }
#undef GDN_SC
  return hipGetLastError();
}

template <int DK>
static void launch_segment_tail(const SegArgs& seg, void* o, float* ST, int B,
                                int T, int H, int dv, hipStream_t stream) {
  hipLaunchKernelGGL((segment_combine_kernel<DK>), dim3(B * H * (dv / 16)),
                     dim3(64 * (DK / 16 + 1)), 0, stream, seg, ST, dv);
  const dim3 grid(B * H * (seg.nseg - 1));
  if (dv == 128)
    hipLaunchKernelGGL((segment_correct_kernel<DK, 128>), grid,
                       dim3(64 * (128 / 16 + kCorrLoaders)), 0, stream, seg,
                       static_cast<bf16*>(o), T, H);
  else
    hipLaunchKernelGGL((segment_correct_kernel<DK, 64>), grid,
                       dim3(64 * (64 / 16 + kCorrLoaders)), 0, stream, seg,
                       static_cast<bf16*>(o), T, H);
}

hipError_t launch_prefill_scan(const void* q, const void* k, const void* v,
                               const float* S0, void* o, float* ST, void* ws,
                               int B, int T, int H, int dk, int dv,
                               int in_dtype, int out_dtype, hipStream_t stream) {
  const bool ib = in_dtype == 1, ob = out_dtype == 1;
  const PrefillPlan plan = plan_prefill(B, T, H, dk, dv);
  SegArgs seg{};
  seg.nseg = 1;
  seg.seg_chunks = plan.nchunks;
  char* wsb = static_cast<char*>(ws);
  if (plan.nseg > 1 && ib && ob) {
    seg.nseg = plan.nseg;
    seg.seg_chunks = plan.seg_chunks;
    seg.xhat = wsb + plan.xhat_off;
    seg.S_fin = reinterpret_cast<float*>(wsb + plan.sfin_off);
    seg.X_fin = wsb + plan.xfin_off;
    seg.S_in = wsb + plan.sin_off;
  }
  const float* wsf = static_cast<const float*>(ws);
#define GDN_SCAN(DK, TI, TO) \
  launch_scan_t<DK, TI, TO>(q, k, v, S0, o, ST, wsf, B, T, H, dv, seg, stream)
  if (dk == 128) {
    if (ib && ob) GDN_SCAN(128, bf16, bf16);
    else if (ib) GDN_SCAN(128, bf16, float);
    else if (ob) GDN_SCAN(128, float, bf16);
    else GDN_SCAN(128, float, float);
  } else {
    if (ib && ob) GDN_SCAN(64, bf16, bf16);
    else if (ib) GDN_SCAN(64, bf16, float);
    else if (ob) GDN_SCAN(64, float, bf16);
    else GDN_SCAN(64, float, float);
  }
#undef GDN_SCAN
  if (seg.nseg > 1) {
    if (dk == 128) launch_segment_tail<128>(seg, o, ST, B, T, H, dv, stream);
    else launch_segment_tail<64>(seg, o, ST, B, T, H, dv, stream);
  }
  return hipGetLastError();
}

}  // namespace gdn
