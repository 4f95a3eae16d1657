// Chunked prefill of the gated delta rule on gfx950.
//
// The token recurrence (decay, predict with the decayed state, delta write,
// read the new state; "On State Reduction in Linear Attention", Sec. 2.1,
// Eq. (2) with gated decay, and "Linear Attention Architectures", Sec. 3.3)
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
// This is an exact re-association of the sequential recurrence.
//
// Two kernels:
//  * prepare_kernel -- one workgroup per (batch, head, chunk), fully
//    parallel: gate prefix sums, K K^T and Q K^T on bf16 MFMA, the
//    triangular inverse T by forward substitution in fp32; writes T, P and
//    the gate block to the workspace.
//  * scan_kernel -- one workgroup per (batch, head, 16 state rows); the rows
//    of the state evolve independently ("On State Reduction in Linear
//    Attention", Sec. 3.1), so each workgroup carries a 16 x dk slice of S in
//    MFMA accumulators and walks the chunks in order.  Every product that
//    touches the state uses split-bf16 operands (x = hi + lo, three or two
//    MFMAs) so the carried state keeps ~16 significant bits per operand and
//    fp32 accumulation; outputs stored in bf16 use single-pass products.
//    The next chunk's tiles are prefetched into registers while the current
//    chunk computes.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int C = kChunk;

// The 10 lower-triangular 16x16 tiles (mi >= ni) of a 64x64 matrix.
__device__ __constant__ int kLowerMi[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__device__ __constant__ int kLowerNi[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

// k-slot j (0..7) of lane group g4 inside 32-wide k-block s.  A lane's slots
// are two runs of 4 consecutive indices, which matches how an MFMA
// accumulator tile holds its rows (4 consecutive rows per lane group), so
// results can be fed back as B operands without any transpose.
__device__ __forceinline__ int kslot_base(int s, int g4, int half) {
  return 32 * s + 16 * half + 4 * g4;
}

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float* x) {
  const float4 a = load4(p), b = load4(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

}  // namespace

// ===========================================================================
// prepare
// ===========================================================================

template <int DK, typename TIn>
__global__ __launch_bounds__(256) void prepare_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ ws, int T, int H, int nchunks) {
  constexpr bool SPLIT = std::is_same<TIn, float>::value;  // inputs not bf16
  constexpr int LD = DK + 8;            // bf16 row stride of the K/Q tiles
  constexpr int LDA = C + 4;            // fp32 row stride of A
  __shared__ __attribute__((aligned(16))) bf16 Kh[C * LD];
  __shared__ __attribute__((aligned(16))) bf16 Qh[C * LD];
  __shared__ __attribute__((aligned(16))) bf16 Kl[SPLIT ? C * LD : 8];
  __shared__ __attribute__((aligned(16))) bf16 Ql[SPLIT ? C * LD : 8];
  __shared__ __attribute__((aligned(16))) float As[C * LDA];
  __shared__ float gs[C], bs[C];

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = chunk * C;
  const int nvalid = min(C, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* wsc = ws + ((size_t)(b * H + h) * nchunks + chunk) * kChunkWsFloats;
  float* Tw = wsc;
  float* Pw = wsc + C * C;
  float* Gw = wsc + 2 * C * C;

  // 1. stage K and Q (zero rows past the end of the sequence)
  constexpr int SEGS = C * DK / 8;
  for (int sg = tid; sg < SEGS; sg += 256) {
    const int c = sg / (DK / 8), d0 = (sg % (DK / 8)) * 8;
    float kx[8], qx[8];
    if (c < nvalid) {
      const size_t off = (((size_t)b * T + t0 + c) * H + h) * DK + d0;
      load8(k + off, kx);
      load8(q + off, qx);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kx[e] = qx[e] = 0.f;
    }
    bf16x8 kh, qh;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kh[e] = (bf16)kx[e];
      qh[e] = (bf16)qx[e];
    }
    *reinterpret_cast<bf16x8*>(&Kh[c * LD + d0]) = kh;
    *reinterpret_cast<bf16x8*>(&Qh[c * LD + d0]) = qh;
    if constexpr (SPLIT) {
      bf16x8 kl, ql;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kl[e] = (bf16)(kx[e] - (float)kh[e]);
        ql[e] = (bf16)(qx[e] - (float)qh[e]);
      }
      *reinterpret_cast<bf16x8*>(&Kl[c * LD + d0]) = kl;
      *reinterpret_cast<bf16x8*>(&Ql[c * LD + d0]) = ql;
    }
  }

  // 2. gates: inclusive prefix sum of log alpha inside the chunk
  if (w == 0) {
    float a = 1.f, be = 0.f;                  // padding tokens: identity step
    if (lane < nvalid) {
      const size_t gi = ((size_t)b * T + t0 + lane) * H + h;
      a = alpha[gi];
      be = beta[gi];
    }
    float g = logf(a);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(g, off, 64);
      if (lane >= off) g += y;
    }
    const float glast = __shfl(g, 63, 64);
    gs[lane] = g;
    bs[lane] = be;
    Gw[lane] = g;
    Gw[C + lane] = be;
    Gw[2 * C + lane] = expf(g);
    Gw[3 * C + lane] = expf(glast - g);
  }
  // upper-triangle tiles of P are zero
  for (int e = tid; e < C * C; e += 256) {
    const int j = e / C, i = e % C;
    if ((i >> 4) > (j >> 4)) Pw[e] = 0.f;
  }
  __syncthreads();

  // 3. lower tiles of K K^T (-> A) and Q K^T (-> P), 20 tiles over 4 waves
  const int n = lane & 15, g4 = lane >> 4;
  for (int t = w; t < 20; t += 4) {
    const bool isP = t >= 10;
    const int mi = kLowerMi[isP ? t - 10 : t], ni = kLowerNi[isP ? t - 10 : t];
    const bf16* Xh = isP ? Qh : Kh;
    const bf16* Xl = isP ? Ql : Kl;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const int col = 32 * s + 8 * g4;
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Xh[(16 * mi + n) * LD + col]);
      const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&Kh[(16 * ni + n) * LD + col]);
      acc = mfma(ah, bh, acc);
      if constexpr (SPLIT) {
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Xl[(16 * mi + n) * LD + col]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&Kl[(16 * ni + n) * LD + col]);
        acc = mfma(ah, bl, acc);
        acc = mfma(al, bh, acc);
      }
    }
    const int i = 16 * ni + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 16 * mi + 4 * g4 + e;
      const float decay = expf(gs[j] - gs[i]);
      if (isP) {
        Pw[j * C + i] = (i <= j) ? decay * acc[e] : 0.f;
      } else {
        As[j * LDA + i] = (i < j) ? bs[j] * decay * acc[e] : 0.f;
      }
    }
  }
  __syncthreads();

  // 4. T = (I + A)^{-1} by forward substitution, one column per lane
  if (w == 0) {
    const int c = lane;
    float tc[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float acc = (j == c) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < j; ++i) acc -= As[j * LDA + i] * tc[i];
      tc[j] = acc;
    }
#pragma unroll
    for (int j = 0; j < C; ++j) Tw[j * C + c] = tc[j];
  }
}

// ===========================================================================
// scan
// ===========================================================================

template <int DK, typename TIn>
struct Stage {
  static constexpr int UNITS_K = C * DK * (int)sizeof(TIn) / 16 / 256;  // 16B units/thread
  uint4 k[UNITS_K];
  uint4 q[UNITS_K];
  float4 t[4];
  float4 p[4];
  float4 v;          // 4 values of the V slice (bf16 inputs use .x/.y bits)
  float g;
};

template <int DK, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void scan_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* S0, TOut* __restrict__ o,
    float* ST, const float* __restrict__ ws, int T, int H, int DV,
    int nchunks, int nblocks) {
  constexpr bool KEXACT = std::is_same<TIn, bf16>::value;   // q, k, v exact in bf16
  constexpr bool OPREC = std::is_same<TOut, float>::value;  // o stored in fp32
  using KT = typename std::conditional<KEXACT, bf16, float>::type;
  constexpr int LDK = KEXACT ? DK + 8 : DK + 4;   // K/Q tile row stride
  constexpr int LDT = C + 8;                      // bf16 stride of T/P
  constexpr int LDV = C + 4;                      // fp32 stride of [r][c] tiles
  constexpr int LDS_ = DK + 4;                    // fp32 stride of the S slice
  constexpr int NDT = DK / 64;                    // state d-tiles per wave
  constexpr int EPU = 16 / (int)sizeof(TIn);      // elements per 16B unit
  constexpr int UPR = DK / EPU;                   // 16B units per K/Q row
  using St = Stage<DK, TIn>;

  __shared__ __attribute__((aligned(16))) KT Ks[C * LDK];
  __shared__ __attribute__((aligned(16))) KT Qs[C * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Th[C * LDT];
  __shared__ __attribute__((aligned(16))) bf16 Tl[C * LDT];
  __shared__ __attribute__((aligned(16))) bf16 Ph[C * LDT];
  __shared__ __attribute__((aligned(16))) bf16 Pl[OPREC ? C * LDT : 8];
  __shared__ __attribute__((aligned(16))) float Vt[16 * LDV];
  __shared__ __attribute__((aligned(16))) float Gs[4 * C];
  __shared__ __attribute__((aligned(16))) float Sx[16 * LDS_];
  __shared__ __attribute__((aligned(16))) float Zt[16 * LDV];
  __shared__ __attribute__((aligned(16))) float Ut[16 * LDV];

  // workgroup -> (head, 16-row slice); the slices of one head are placed on
  // one XCD (workgroups are dealt to the 8 XCDs round-robin) so they share
  // that XCD's L2 copy of the chunk tiles.
  int lin = blockIdx.x;
  if ((nblocks & 7) == 0) lin = (lin & 7) * (nblocks >> 3) + (lin >> 3);
  const int NS = DV / 16;
  const int bh = lin / NS, slice = lin - bh * NS;
  const int b = bh / H, h = bh - b * H;
  const int r0 = slice * 16;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;

  // ---- stage helpers ----
  auto load_stage = [&](St& st, int chunk) {
    const int t0 = chunk * C;
    const int nvalid = min(C, T - t0);
#pragma unroll
    for (int i = 0; i < St::UNITS_K; ++i) {
      const int u = tid + 256 * i;
      const int c = u / UPR, cu = u - c * UPR;
      // (written as two plain stores: a chained assignment here crashes the
      // ROCm 7.2 backend's machine copy propagation)
      st.k[i] = make_uint4(0, 0, 0, 0);
      st.q[i] = make_uint4(0, 0, 0, 0);
      if (c < nvalid) {
        const size_t row = (((size_t)b * T + t0 + c) * H + h) * DK;
        st.k[i] = *reinterpret_cast<const uint4*>(k + row + cu * EPU);
        st.q[i] = *reinterpret_cast<const uint4*>(q + row + cu * EPU);
      }
    }
    const float* wsc = ws + ((size_t)bh * nchunks + chunk) * kChunkWsFloats;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.t[i] = *reinterpret_cast<const float4*>(wsc + 4 * (tid + 256 * i));
      st.p[i] = *reinterpret_cast<const float4*>(wsc + C * C + 4 * (tid + 256 * i));
    }
    st.g = wsc[2 * C * C + tid];
    const int c = tid >> 2, r4 = (tid & 3) * 4;
    if (c < nvalid) {
      st.v = load4(v + (((size_t)b * T + t0 + c) * H + h) * DV + r0 + r4);
    } else {
      st.v = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  auto commit_stage = [&](const St& st) {
#pragma unroll
    for (int i = 0; i < St::UNITS_K; ++i) {
      const int u = tid + 256 * i;
      const int c = u / UPR, cu = u - c * UPR;
      *reinterpret_cast<uint4*>(&Ks[c * LDK + cu * EPU]) = st.k[i];
      *reinterpret_cast<uint4*>(&Qs[c * LDK + cu * EPU]) = st.q[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e0 = 4 * (tid + 256 * i);
      const int j = e0 / C, i0 = e0 - j * C;
      bf16x4 th, tl, ph, pl;
      const float tv[4] = {st.t[i].x, st.t[i].y, st.t[i].z, st.t[i].w};
      const float pv[4] = {st.p[i].x, st.p[i].y, st.p[i].z, st.p[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        th[e] = (bf16)tv[e];
        tl[e] = (bf16)(tv[e] - (float)th[e]);
        ph[e] = (bf16)pv[e];
        pl[e] = (bf16)(pv[e] - (float)ph[e]);
      }
      *reinterpret_cast<bf16x4*>(&Th[j * LDT + i0]) = th;
      *reinterpret_cast<bf16x4*>(&Tl[j * LDT + i0]) = tl;
      *reinterpret_cast<bf16x4*>(&Ph[j * LDT + i0]) = ph;
      if constexpr (OPREC) *reinterpret_cast<bf16x4*>(&Pl[j * LDT + i0]) = pl;
    }
    const int c = tid >> 2, r4 = (tid & 3) * 4;
    Vt[(r4 + 0) * LDV + c] = st.v.x;
    Vt[(r4 + 1) * LDV + c] = st.v.y;
    Vt[(r4 + 2) * LDV + c] = st.v.z;
    Vt[(r4 + 3) * LDV + c] = st.v.w;
    Gs[tid] = st.g;
  };

  // A operand: 8 k-slots of row `row` of a K/Q tile (bf16 hi [+ lo]).
  auto read_kq = [&](const KT* X, int row, int s, bf16x8& hi, bf16x8& lo) {
    if constexpr (KEXACT) {
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(&X[row * LDK + kslot_base(s, g4, 0)]);
      const bf16x4 c2 = *reinterpret_cast<const bf16x4*>(&X[row * LDK + kslot_base(s, g4, 1)]);
      hi = __builtin_shufflevector(a, c2, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(&X[row * LDK + kslot_base(s, g4, 0)]);
      const float4 c2 = *reinterpret_cast<const float4*>(&X[row * LDK + kslot_base(s, g4, 1)]);
      const floatx8 x = {a.x, a.y, a.z, a.w, c2.x, c2.y, c2.z, c2.w};
      split8(x, hi, lo);
    }
  };
  // 8 k-slots of an fp32 [r][k] tile at row n (B operand of a k-block).
  auto read_f8 = [&](const float* X, int ld, int s) -> floatx8 {
    const float4 a = *reinterpret_cast<const float4*>(&X[n * ld + kslot_base(s, g4, 0)]);
    const float4 c2 = *reinterpret_cast<const float4*>(&X[n * ld + kslot_base(s, g4, 1)]);
    const floatx8 x = {a.x, a.y, a.z, a.w, c2.x, c2.y, c2.z, c2.w};
    return x;
  };
  // 8 k-slots of row `row` of a bf16 [c][c'] tile.
  auto read_t8 = [&](const bf16* X, int row, int s) -> bf16x8 {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(&X[row * LDT + kslot_base(s, g4, 0)]);
    const bf16x4 c2 = *reinterpret_cast<const bf16x4*>(&X[row * LDT + kslot_base(s, g4, 1)]);
    return __builtin_shufflevector(a, c2, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // ---- carried state: wave w owns d-tiles w*NDT .. w*NDT+NDT-1 ----
  floatx4 accS[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    const int d0 = 16 * (w * NDT + t) + 4 * g4;
    if (S0 != nullptr) {
      const float4 x = *reinterpret_cast<const float4*>(
          S0 + ((size_t)bh * DV + r0 + n) * DK + d0);
      accS[t] = floatx4{x.x, x.y, x.z, x.w};
    } else {
      accS[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  St st;
  load_stage(st, 0);

  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int t0 = chunk * C;
    const int nvalid = min(C, T - t0);
    __syncthreads();                 // previous chunk done with the LDS tiles
    commit_stage(st);
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      const int d0 = 16 * (w * NDT + t) + 4 * g4;
      *reinterpret_cast<float4*>(&Sx[n * LDS_ + d0]) =
          make_float4(accS[t][0], accS[t][1], accS[t][2], accS[t][3]);
    }
    __syncthreads();
    if (chunk + 1 < nchunks) load_stage(st, chunk + 1);   // prefetch

    const int crow = 16 * w + n;         // A-operand row of this wave's c-tile
    const int cacc = 16 * w + 4 * g4;    // first accumulator row (c) of lane

    // ---- Y = K S^T for c-tile w (state-touching: split S) ----
    floatx4 accY = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      bf16x8 ah, al, bh, bl;
      read_kq(Ks, crow, s, ah, al);
      split8(read_f8(Sx, LDS_, s), bh, bl);
      accY = mfma(ah, bh, accY);
      accY = mfma(ah, bl, accY);
      if constexpr (!KEXACT) accY = mfma(al, bh, accY);
    }

    // ---- Z = beta (V - gamma Y) -> Zt[r][c] ----
    {
      const float4 vv = *reinterpret_cast<const float4*>(&Vt[n * LDV + cacc]);
      const float4 bb = *reinterpret_cast<const float4*>(&Gs[C + cacc]);
      const float4 gg = *reinterpret_cast<const float4*>(&Gs[2 * C + cacc]);
      float4 z;
      z.x = bb.x * (vv.x - gg.x * accY[0]);
      z.y = bb.y * (vv.y - gg.y * accY[1]);
      z.z = bb.z * (vv.z - gg.z * accY[2]);
      z.w = bb.w * (vv.w - gg.w * accY[3]);
      *reinterpret_cast<float4*>(&Zt[n * LDV + cacc]) = z;
    }
    __syncthreads();

    // ---- U = T Z for c-tile w (T lower triangular: k-blocks <= w/2) ----
    floatx4 accU = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s <= (w >> 1); ++s) {
      const bf16x8 th = read_t8(Th, crow, s), tl = read_t8(Tl, crow, s);
      bf16x8 zh, zl;
      split8(read_f8(Zt, LDV, s), zh, zl);
      accU = mfma(th, zh, accU);
      accU = mfma(th, zl, accU);
      accU = mfma(tl, zh, accU);
    }
    *reinterpret_cast<float4*>(&Ut[n * LDV + cacc]) =
        make_float4(accU[0], accU[1], accU[2], accU[3]);
    __syncthreads();

    // ---- O = diag(gamma) Q S^T + P U for c-tile w ----
    {
      floatx4 accO = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        bf16x8 ah, al, bh, bl;
        read_kq(Qs, crow, s, ah, al);
        split8(read_f8(Sx, LDS_, s), bh, bl);
        accO = mfma(ah, bh, accO);
        if constexpr (OPREC) {
          accO = mfma(ah, bl, accO);
          if constexpr (!KEXACT) accO = mfma(al, bh, accO);
        }
      }
      const float4 gg = *reinterpret_cast<const float4*>(&Gs[2 * C + cacc]);
      accO[0] *= gg.x;
      accO[1] *= gg.y;
      accO[2] *= gg.z;
      accO[3] *= gg.w;
      for (int s = 0; s <= (w >> 1); ++s) {
        const bf16x8 ph = read_t8(Ph, crow, s);
        bf16x8 uh, ul;
        split8(read_f8(Ut, LDV, s), uh, ul);
        accO = mfma(ph, uh, accO);
        if constexpr (OPREC) {
          const bf16x8 pl = read_t8(Pl, crow, s);
          accO = mfma(ph, ul, accO);
          accO = mfma(pl, uh, accO);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = cacc + e;
        if (c < nvalid)
          store1(o + (((size_t)b * T + t0 + c) * H + h) * DV + r0 + n, accO[e]);
      }
    }

    // ---- S^T <- gamma_C S^T + K^T diag(e^{g_C - g}) U  (owned d-tiles) ----
    {
      const float gC = Gs[2 * C + C - 1];
      bf16x8 uh[2], ul[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const floatx8 u8 = read_f8(Ut, LDV, s);
        const float4 d0 = *reinterpret_cast<const float4*>(&Gs[3 * C + kslot_base(s, g4, 0)]);
        const float4 d1 = *reinterpret_cast<const float4*>(&Gs[3 * C + kslot_base(s, g4, 1)]);
        const floatx8 du = {u8[0] * d0.x, u8[1] * d0.y, u8[2] * d0.z, u8[3] * d0.w,
                            u8[4] * d1.x, u8[5] * d1.y, u8[6] * d1.z, u8[7] * d1.w};
        split8(du, uh[s], ul[s]);
      }
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        const int dcol = 16 * (w * NDT + t) + n;   // A row = state column d
        floatx4 acc = accS[t] * gC;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          floatx8 kx;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kx[e] = (float)Ks[(kslot_base(s, g4, 0) + e) * LDK + dcol];
            kx[4 + e] = (float)Ks[(kslot_base(s, g4, 1) + e) * LDK + dcol];
          }
          bf16x8 kh, kl;
          if constexpr (KEXACT) {
            kh = to_bf16x8(kx);
          } else {
            split8(kx, kh, kl);
          }
          acc = mfma(kh, uh[s], acc);
          acc = mfma(kh, ul[s], acc);
          if constexpr (!KEXACT) acc = mfma(kl, uh[s], acc);
        }
        accS[t] = acc;
      }
    }
  }

  if (ST != nullptr) {
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      const int d0 = 16 * (w * NDT + t) + 4 * g4;
      *reinterpret_cast<float4*>(ST + ((size_t)bh * DV + r0 + n) * DK + d0) =
          make_float4(accS[t][0], accS[t][1], accS[t][2], accS[t][3]);
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

template <int DK, typename TIn>
static void launch_prepare_t(const void* q, const void* k, const float* alpha,
                             const float* beta, float* ws, int B, int T, int H,
                             hipStream_t stream) {
  const int nchunks = (T + C - 1) / C;
  hipLaunchKernelGGL((prepare_kernel<DK, TIn>), dim3(nchunks, H, B), dim3(256),
                     0, stream, static_cast<const TIn*>(q),
                     static_cast<const TIn*>(k), alpha, beta, ws, T, H,
                     nchunks);
}

hipError_t launch_prefill_prepare(const void* q, const void* k,
                                  const float* alpha, const float* beta,
                                  float* ws, int B, int T, int H, int dk,
                                  int in_dtype, hipStream_t stream) {
  if (in_dtype == 1) {
    if (dk == 128) launch_prepare_t<128, bf16>(q, k, alpha, beta, ws, B, T, H, stream);
    else launch_prepare_t<64, bf16>(q, k, alpha, beta, ws, B, T, H, stream);
  } else {
    if (dk == 128) launch_prepare_t<128, float>(q, k, alpha, beta, ws, B, T, H, stream);
    else launch_prepare_t<64, float>(q, k, alpha, beta, ws, B, T, H, stream);
  }
  return hipGetLastError();
}

template <int DK, typename TIn, typename TOut>
static void launch_scan_t(const void* q, const void* k, const void* v,
                          const float* S0, void* o, float* ST, const float* ws,
                          int B, int T, int H, int dv, hipStream_t stream) {
  const int nchunks = (T + C - 1) / C;
  const int nblocks = B * H * (dv / 16);
  hipLaunchKernelGGL((scan_kernel<DK, TIn, TOut>), dim3(nblocks), dim3(256), 0,
                     stream, static_cast<const TIn*>(q),
                     static_cast<const TIn*>(k), static_cast<const TIn*>(v),
                     S0, static_cast<TOut*>(o), ST, ws, T, H, dv, nchunks,
                     nblocks);
}

hipError_t launch_prefill_scan(const void* q, const void* k, const void* v,
                               const float* S0, void* o, float* ST,
                               const float* ws, int B, int T, int H, int dk,
                               int dv, int in_dtype, int out_dtype,
                               hipStream_t stream) {
#define GDN_SCAN(DK, TI, TO) \
  launch_scan_t<DK, TI, TO>(q, k, v, S0, o, ST, ws, B, T, H, dv, stream)
  const bool ib = in_dtype == 1, ob = out_dtype == 1;
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
  return hipGetLastError();
}

}  // namespace gdn
