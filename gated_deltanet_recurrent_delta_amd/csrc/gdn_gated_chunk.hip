// Generalised gates in chunked form, on gfx950.
//
// The recurrence ("Linear Attention Architectures" reading notes on paper
// Sec. 3.4, Kimi Delta Attention, and Sec. 3.5, Gated DeltaNet-2): per head
// and token, with a retention a_t per KEY channel, a key-side erase gate b_t
// and a value-side write gate w_t,
//     S~ = S_{t-1} diag(a_t),  e_t = b_t * k_t,  z_t = w_t * v_t,
//     S_t = S~ (I - e_t k_t^T) + z_t k_t^T = S~ + u_t k_t^T,
//     u_t = z_t - S~ e_t,        o_t = S_t q_t.
// Inside a chunk of 64 tokens with incoming state S and the per-channel
// cumulative log retention G_j = sum_{m <= j} log a_m (a vector over the
// key channels), unrolling gives (all exact):
//     A_ji = sum_d e_jd k_id e^{G_jd - G_id}   (i < j),  T = (I + A)^{-1}
//     P_ji = sum_d q_jd k_id e^{G_jd - G_id}   (i <= j)
//     U = T (Z - K~ S^T),  K~_j = e_j * e^{G_j},  Z_j = z_j
//     O = Q~ S^T + P U,    Q~_j = q_j * e^{G_j}
//     S' = S diag(e^{G_C}) + U^T K^,  K^_i = k_i * e^{G_C - G_i}.
// Every exponent in K~, Q~ and K^ is <= 0.  A and P contract over the key
// channels with a decay ratio per channel, so they are formed as products
// of decay-weighted factors: the rows of row block jb (16 tokens) are
// weighted against a reference token r = 16 jb + 8 (the block's middle),
//     e_jd e^{G_jd - G_rd}  and  k_id e^{G_rd - G_id},
// whose exponents span at most 8 tokens of decay above zero (for i, j in
// the block) and are <= 0 otherwise, so no factor over- or underflows for
// per-token log2 retentions down to about -15 (retention 3e-5 per token).
//
// The kernels:
//  * gated_prepare_kernel -- one workgroup (4 waves) per (batch, head,
//    chunk): per-channel prefix sums of log2 a; K~, Q~, K^ (split bf16 hi /
//    lo) and e^{G_C} to the workspace; the 16x16 tiles of A and P on bf16
//    MFMA with split operands (wave = row block); T = (I + A)^{-1} in fp32
//    (diagonal blocks by forward substitution, then the off-diagonal blocks
//    level by level); T and P to the workspace as split bf16 tiles in the
//    layout the plain prefill uses.
//  * gated_scan_kernel -- one workgroup per (batch, head, 64 state rows),
//    sequential over the chunks; wave w carries 16 state rows as S^T
//    accumulator tiles (rows independent, "On State Reduction in Linear
//    Attention", paper Sec. 3.1) and does the chunk step with split-bf16
//    operands throughout (three MFMAs per product): K~, Q~, K^ are not
//    exact bf16 and the state is fp32.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include "gdn_tiles.hpp"

namespace gdn {

namespace {

// Workspace of one (batch, head, chunk), in bytes: the T / P tiles at the
// plain prefill's offsets (kWsTh .. kWsPl), then K~ hi, K~ lo, Q~ hi, Q~ lo,
// K^ hi, K^ lo (bf16 [64][dk] each), then e^{G_C} (fp32 [dk]).
constexpr int kGOffOps = 32768;
__host__ __device__ constexpr size_t gated_chunk_bytes(int dk) {
  return (size_t)kGOffOps + 6 * (size_t)C * dk * 2 + (size_t)dk * 4;
}

__device__ __forceinline__ floatx8 f8(const float (&x)[8]) {
  const floatx8 r = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return r;
}

}  // namespace

size_t gated_chunked_ws_bytes(int B, int T, int H, int dk) {
  return (size_t)B * H * ((T + C - 1) / C) * gated_chunk_bytes(dk);
}

// ===========================================================================
// prepare
// ===========================================================================

// LO: also the lo parts of Q~ and P, which only fp32 outputs use (bf16
// outputs take single-pass Q~ S^T and P U, as the plain prefill does).
template <int DK, bool LO>
__global__ __launch_bounds__(256) void gated_prepare_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k,
    const float* __restrict__ alpha, const float* __restrict__ bgate,
    char* __restrict__ ws, int T, int H, int nchunks) {
  constexpr int NT = 256;
  constexpr int NKB = DK / 32;
  constexpr int LG = DK + 1;           // fp32 row stride: rows on different banks
  constexpr int LKB = DK + 8;          // bf16 row stride of K, Q
  constexpr int LA = C + 1;            // fp32 row stride of A, P, T
  __shared__ float G2[C * LG];         // log2 a, then its prefix over tokens; later T
  __shared__ float Ef[C * LG];         // e = b * k; later A
  __shared__ __attribute__((aligned(16))) bf16 Kb[C * LKB];
  __shared__ __attribute__((aligned(16))) bf16 Qb[C * LKB];
  __shared__ float Pm[C * LA];
  __shared__ float Wt[16 * 17];
  __shared__ float part[4 * DK];       // per-quarter sums of the prefix
  static_assert(C * LA <= C * LG, "T and A fit in the prefix-sum and e buffers");
  float* Tm = G2;                      // after the A / P operands are formed
  float* Am = Ef;                      // likewise

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = chunk * C, nvalid = min(C, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  char* wsc = ws + ((size_t)(b * H + h) * nchunks + chunk) * gated_chunk_bytes(DK);

  // 1. gates and inputs, four channels per thread and unit; tokens past
  //    the end are identity steps (a = 1, b = k = q = 0).  Every load is
  //    issued first, unconditionally (rows clamped to the last token), then
  //    masked: a load under a branch would make each wait drain them all.
  constexpr int NU1 = C * DK / 4 / NT;
  static_assert(NU1 * NT * 4 == C * DK, "whole units per thread");
  float4 ra[NU1], rb[NU1];
  uint2 rk[NU1], rq[NU1];
#pragma unroll
  for (int i = 0; i < NU1; ++i) {
    const int u = tid + NT * i, j = u / (DK / 4), d = (u - j * (DK / 4)) * 4;
    const size_t off = (((size_t)b * T + t0 + min(j, nvalid - 1)) * H + h) * DK + d;
    ra[i] = *reinterpret_cast<const float4*>(alpha + off);
    rb[i] = *reinterpret_cast<const float4*>(bgate + off);
    rk[i] = *reinterpret_cast<const uint2*>(k + off);
    rq[i] = *reinterpret_cast<const uint2*>(q + off);
  }
#pragma unroll
  for (int i = 0; i < NU1; ++i) {
    const int u = tid + NT * i, j = u / (DK / 4), d = (u - j * (DK / 4)) * 4;
    const bool ok = j < nvalid;
    const uint32_t mk = ok ? 0xFFFFFFFFu : 0u;
    const uint2 kk = make_uint2(rk[i].x & mk, rk[i].y & mk), qq = make_uint2(rq[i].x & mk, rq[i].y & mk);
    const float4 a4 = ra[i], b4 = rb[i];
    const float la[4] = {ok ? log2f(a4.x) : 0.f, ok ? log2f(a4.y) : 0.f,
                         ok ? log2f(a4.z) : 0.f, ok ? log2f(a4.w) : 0.f};
    const float bb[4] = {ok ? b4.x : 0.f, ok ? b4.y : 0.f, ok ? b4.z : 0.f, ok ? b4.w : 0.f};
    const float kf[4] = {bf16lo(kk.x), bf16hi(kk.x), bf16lo(kk.y), bf16hi(kk.y)};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      G2[j * LG + d + x] = la[x];
      Ef[j * LG + d + x] = bb[x] * kf[x];
    }
    *reinterpret_cast<uint2*>(&Kb[j * LKB + d]) = kk;
    *reinterpret_cast<uint2*>(&Qb[j * LKB + d]) = qq;
  }
  __syncthreads();
  // inclusive prefix over the tokens: four quarters of 16 tokens per
  // channel, then each quarter adds the totals of those before it
  for (int u = tid; u < 4 * DK; u += NT) {
    const int d = u % DK, qt = u / DK;
    float g = 0.f;
    for (int j = 16 * qt; j < 16 * qt + 16; ++j) {
      g += G2[j * LG + d];
      G2[j * LG + d] = g;
    }
    part[qt * DK + d] = g;
  }
  __syncthreads();
  for (int u = tid; u < 3 * 16 * DK; u += NT) {
    const int qt = 1 + u / (16 * DK), rem = u - (qt - 1) * 16 * DK;
    const int j = 16 * qt + rem / DK, d = rem % DK;
    float off = 0.f;
    for (int p = 0; p < qt; ++p) off += part[p * DK + d];
    G2[j * LG + d] += off;
  }
  __syncthreads();

  // 2. the scan's operands
  {
    char* kt = wsc + kGOffOps;
    constexpr int MB = C * DK * 2;     // bytes of one [C][DK] bf16 matrix
    for (int u = tid; u < C * DK / 8; u += NT) {
      const int j = u / (DK / 8), d0 = (u - j * (DK / 8)) * 8;
      float a[8], c[8], e[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float g = G2[j * LG + d0 + x], gc = G2[(C - 1) * LG + d0 + x];
        const float f = exp2f(g);
        a[x] = Ef[j * LG + d0 + x] * f;
        c[x] = (float)Qb[j * LKB + d0 + x] * f;
        e[x] = (float)Kb[j * LKB + d0 + x] * exp2f(gc - g);
      }
      bf16x8 hi, lo;
      const size_t o = (size_t)(j * DK + d0) * 2;
      split8(f8(a), hi, lo);
      *reinterpret_cast<bf16x8*>(kt + o) = hi;
      *reinterpret_cast<bf16x8*>(kt + MB + o) = lo;
      split8(f8(c), hi, lo);
      *reinterpret_cast<bf16x8*>(kt + 2 * MB + o) = hi;
      if constexpr (LO) *reinterpret_cast<bf16x8*>(kt + 3 * MB + o) = lo;
      split8(f8(e), hi, lo);
      *reinterpret_cast<bf16x8*>(kt + 4 * MB + o) = hi;
      *reinterpret_cast<bf16x8*>(kt + 5 * MB + o) = lo;
    }
    if (tid < DK)
      reinterpret_cast<float*>(kt + 6 * MB)[tid] = exp2f(G2[(C - 1) * LG + tid]);
  }

  // 3. A and P: wave w forms row block jb = w against reference r
  {
    const int jb = w, r = 16 * jb + 8;
    const int j = 16 * jb + n;                       // A-operand row of this lane
    bf16x8 leh[NKB], lel[NKB], lqh[NKB], lql[NKB];
#pragma unroll
    for (int s = 0; s < NKB; ++s) {
      float le[8], lq[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int d = kslot_base(s, g4, x >> 2) + (x & 3);
        const float f = exp2f(G2[j * LG + d] - G2[r * LG + d]);
        le[x] = Ef[j * LG + d] * f;
        lq[x] = (float)Qb[j * LKB + d] * f;
      }
      split8(f8(le), leh[s], lel[s]);
      split8(f8(lq), lqh[s], lql[s]);
    }
    __syncthreads();                   // every read of e is done: A goes over it
    for (int ib = 0; ib <= jb; ++ib) {
      const int i = 16 * ib + n;                     // B-operand column of this lane
      floatx4 aa = {0.f, 0.f, 0.f, 0.f}, pp = aa;
#pragma unroll
      for (int s = 0; s < NKB; ++s) {
        float rr[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int d = kslot_base(s, g4, x >> 2) + (x & 3);
          rr[x] = (float)Kb[i * LKB + d] * exp2f(G2[r * LG + d] - G2[i * LG + d]);
        }
        bf16x8 rh, rl;
        split8(f8(rr), rh, rl);
        aa = mfma(leh[s], rh, aa);
        aa = mfma(leh[s], rl, aa);
        aa = mfma(lel[s], rh, aa);
        pp = mfma(lqh[s], rh, pp);
        pp = mfma(lqh[s], rl, pp);
        pp = mfma(lql[s], rh, pp);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int jr = 16 * jb + 4 * g4 + x;
        Am[jr * LA + i] = (i < jr) ? aa[x] : 0.f;
        Pm[jr * LA + i] = (i <= jr) ? pp[x] : 0.f;
      }
    }
    for (int ib = jb + 1; ib < 4; ++ib)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int jr = 16 * jb + 4 * g4 + x;
        Am[jr * LA + 16 * ib + n] = 0.f;
        Pm[jr * LA + 16 * ib + n] = 0.f;
      }
  }
  __syncthreads();

  // 4. T = (I + A)^{-1}: diagonal blocks by forward substitution (wave 0,
  //    lane = block g4, column n), then T_ij = -T_ii sum_k A_ik T_kj level
  //    by level (thread = element of the 16x16 block).
  if (w == 0) {
    const int base = 16 * g4, c = n;
    float tcol[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      float acc = (jj == c) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < jj; ++m) acc -= Am[(base + jj) * LA + base + m] * tcol[m];
      tcol[jj] = acc;
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) Tm[(base + jj) * LA + base + c] = tcol[jj];
  }
  __syncthreads();
  {
    const int ii = tid >> 4, jj = tid & 15;
    for (int dist = 1; dist < 4; ++dist) {
      for (int bj = 0; bj + dist < 4; ++bj) {
        const int bi = bj + dist;
        float acc = 0.f;
        for (int bk = bj; bk < bi; ++bk)
#pragma unroll
          for (int m = 0; m < 16; ++m)
            acc += Am[(16 * bi + ii) * LA + 16 * bk + m] * Tm[(16 * bk + m) * LA + 16 * bj + jj];
        Wt[ii * 17 + jj] = acc;
        __syncthreads();
        float t = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) t += Tm[(16 * bi + ii) * LA + 16 * bi + m] * Wt[m * 17 + jj];
        Tm[(16 * bi + ii) * LA + 16 * bj + jj] = -t;
        __syncthreads();
      }
    }
  }

  // 5. T and P -> workspace as bf16 hi/lo tiles: lower 16x16 blocks, zeros
  //    in the upper blocks (0,1) and (2,3); rows 0..31, columns 32..63 are
  //    never read and stay unwritten
  for (int e = tid; e < C * C / 8; e += NT) {
    const int j = (8 * e) / C, i0 = (8 * e) % C;
    if (j < C / 2 && i0 >= C / 2) continue;
    const bool upper = (i0 >> 4) > (j >> 4);
    float tv[8], pv[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      tv[x] = upper ? 0.f : Tm[j * LA + i0 + x];
      pv[x] = Pm[j * LA + i0 + x];
    }
    bf16x8 hi, lo;
    split8(f8(tv), hi, lo);
    *reinterpret_cast<bf16x8*>(wsc + kWsTh + (j * C + i0) * 2) = hi;
    *reinterpret_cast<bf16x8*>(wsc + kWsTl + (j * C + i0) * 2) = lo;
    split8(f8(pv), hi, lo);
    *reinterpret_cast<bf16x8*>(wsc + kWsPh + (j * C + i0) * 2) = hi;
    if constexpr (LO) *reinterpret_cast<bf16x8*>(wsc + kWsPl + (j * C + i0) * 2) = lo;
  }
}

// ===========================================================================
// scan
// ===========================================================================

template <int DK, typename TOut>
__global__ __launch_bounds__(256, 1) void gated_scan_kernel(
    const bf16* __restrict__ v, const float* __restrict__ wgate,
    const float* S0, TOut* __restrict__ o, float* ST,
    const char* __restrict__ ws, int T, int H, int DV, int nchunks, int nblocks) {
  constexpr int NT = 256, ROWS = 64;
  constexpr int LDK = DK + 8, LDT = C + 8;
  constexpr int NDT = DK / 16, NKB = DK / 32;
  constexpr int MB = C * DK * 2;
  constexpr bool OPREC = std::is_same<TOut, float>::value;   // fp32 outputs
  // staged [C][DK] matrices (K~ h/l, Q~ h[/l], K^ h/l) and 64x64 tiles
  // (T h/l, P h[/l]): bf16 outputs skip the lo parts of Q~ and P
  constexpr int NKM = OPREC ? 6 : 5, NTM = OPREC ? 4 : 3;
  __shared__ __attribute__((aligned(16))) bf16 KT[6][C * LDK];   // K~ h/l, Q~ h/l, K^ h/l
  __shared__ __attribute__((aligned(16))) bf16 TP[NTM][C * LDT];  // T h/l, P h[/l]
  __shared__ float LC[DK];

  int lin = blockIdx.x;
  if ((nblocks & 7) == 0) lin = (lin & 7) * (nblocks >> 3) + (lin >> 3);
  const int NRG = DV / ROWS;
  const int bh = lin / NRG, rg = lin - bh * NRG;
  const int b = bh / H, h = bh - b * H;
  const int r0 = rg * ROWS;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g4 = lane >> 4;
  const int row = r0 + 16 * w + n;       // this lane's state row (value channel)

  floatx4 S[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    if (S0 != nullptr) {
      const float4 x = *reinterpret_cast<const float4*>(S0 + ((size_t)bh * DV + row) * DK + 16 * dt + 4 * g4);
      S[dt] = floatx4{x.x, x.y, x.z, x.w};
    } else {
      S[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // The next chunk's tiles and gates are loaded into registers while this
  // chunk computes, and committed to LDS at the top of the next step.
  constexpr int NKT = NKM * C * DK / 8 / NT, NTP = NTM * C * C / 8 / NT;
  static_assert(NKT * NT * 8 == NKM * C * DK && NTP * NT * 8 == NTM * C * C,
                "whole units per thread");
  // staged matrix m' -> workspace / LDS matrix (bf16 outputs skip Q~ lo)
  auto kmat = [](int mp) { return OPREC ? mp : mp + (mp >= 3); };
  struct {
    u32x4 kt[NKT], tp[NTP];
    float lc, w[4][4];
    bf16 v[4][4];
  } st;
  st.lc = 0.f;
  auto load = [&](int chunk) {
    const int t0 = chunk * C, nvalid = min(C, T - t0);
    const char* wsc = ws + ((size_t)bh * nchunks + chunk) * gated_chunk_bytes(DK);
#pragma unroll
    for (int i = 0; i < NKT; ++i) {
      const int u = tid + i * NT;
      const int mp = u / (C * DK / 8), rem = u - mp * (C * DK / 8);
      st.kt[i] = *reinterpret_cast<const u32x4*>(wsc + kGOffOps + kmat(mp) * MB + rem * 16);
    }
#pragma unroll
    for (int i = 0; i < NTP; ++i) {
      const int u = tid + i * NT;
      st.tp[i] = *reinterpret_cast<const u32x4*>(wsc + u * 16);
    }
    if (tid < DK) st.lc = reinterpret_cast<const float*>(wsc + kGOffOps + 6 * MB)[tid];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int c = 16 * ct + 4 * g4 + x;
        const size_t off = (((size_t)b * T + t0 + min(c, nvalid - 1)) * H + h) * DV + row;
        st.w[ct][x] = c < nvalid ? wgate[off] : 0.f;
        st.v[ct][x] = c < nvalid ? v[off] : bf16(0.f);
      }
  };
  load(0);                             // T >= 1: the entry point returns earlier

  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int t0 = chunk * C, nvalid = min(C, T - t0);
    __syncthreads();                   // every read of the last chunk's tiles is done
#pragma unroll
    for (int i = 0; i < NKT; ++i) {
      const int u = tid + i * NT;
      const int mp = u / (C * DK / 8), rem = u - mp * (C * DK / 8);
      const int j = rem / (DK / 8), d0 = (rem - j * (DK / 8)) * 8;
      *reinterpret_cast<u32x4*>(&KT[kmat(mp)][j * LDK + d0]) = st.kt[i];
    }
#pragma unroll
    for (int i = 0; i < NTP; ++i) {
      const int u = tid + i * NT;
      const int m = u / (C * C / 8), rem = u - m * (C * C / 8);
      const int j = rem / (C / 8), i0 = (rem - j * (C / 8)) * 8;
      *reinterpret_cast<u32x4*>(&TP[m][j * LDT + i0]) = st.tp[i];
    }
    if (tid < DK) LC[tid] = st.lc;
    // z = w * v at this lane's tokens (c-tile ct: tokens 16 ct + 4 g4 + x);
    // w is zero past the end
    float z[4][4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int x = 0; x < 4; ++x) z[ct][x] = st.w[ct][x] * (float)st.v[ct][x];
    if (chunk + 1 < nchunks) load(chunk + 1);
    __syncthreads();

    bf16x8 sh[NKB], sl[NKB];
#pragma unroll
    for (int s = 0; s < NKB; ++s) split8(acc_slots(S[2 * s], S[2 * s + 1]), sh[s], sl[s]);
    // Z = z - K~ S^T ;  Q~ S^T
    floatx4 Z[4], OQ[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 y = {0.f, 0.f, 0.f, 0.f}, oq = y;
#pragma unroll
      for (int s = 0; s < NKB; ++s) {
        const bf16x8 kh = lds_slots(KT[0], LDK, 16 * ct + n, s, g4);
        const bf16x8 kl = lds_slots(KT[1], LDK, 16 * ct + n, s, g4);
        const bf16x8 qh = lds_slots(KT[2], LDK, 16 * ct + n, s, g4);
        const bf16x8 ql = OPREC ? lds_slots(KT[3], LDK, 16 * ct + n, s, g4) : bf16x8{};
        y = mfma(kh, sh[s], y);
        y = mfma(kh, sl[s], y);
        y = mfma(kl, sh[s], y);
        oq = mfma(qh, sh[s], oq);
        if constexpr (OPREC) {
          oq = mfma(qh, sl[s], oq);
          oq = mfma(ql, sh[s], oq);
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) Z[ct][x] = z[ct][x] - y[x];
      OQ[ct] = oq;
    }
    // U = T Z  (T lower triangular: k-blocks s <= ct / 2)
    bf16x8 zh[2], zl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) split8(acc_slots(Z[2 * s], Z[2 * s + 1]), zh[s], zl[s]);
    floatx4 U[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= ct / 2; ++s) {
        const bf16x8 th = lds_slots(TP[0], LDT, 16 * ct + n, s, g4);
        const bf16x8 tl = lds_slots(TP[1], LDT, 16 * ct + n, s, g4);
        acc = mfma(th, zh[s], acc);
        acc = mfma(th, zl[s], acc);
        acc = mfma(tl, zh[s], acc);
      }
      U[ct] = acc;
    }
    bf16x8 uh[2], ul[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) split8(acc_slots(U[2 * s], U[2 * s + 1]), uh[s], ul[s]);
    // O = Q~ S^T + P U
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      floatx4 acc = OQ[ct];
#pragma unroll
      for (int s = 0; s <= ct / 2; ++s) {
        const bf16x8 ph = lds_slots(TP[2], LDT, 16 * ct + n, s, g4);
        acc = mfma(ph, uh[s], acc);
        if constexpr (OPREC) {
          const bf16x8 pl = lds_slots(TP[3], LDT, 16 * ct + n, s, g4);
          acc = mfma(ph, ul[s], acc);
          acc = mfma(pl, uh[s], acc);
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int c = 16 * ct + 4 * g4 + x;
        if (c < nvalid) store1(o + (((size_t)b * T + t0 + c) * H + h) * DV + row, acc[x]);
      }
    }
    // S^T <- diag(e^{G_C}) S^T + K^^T U
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float4 lc = *reinterpret_cast<const float4*>(&LC[16 * dt + 4 * g4]);
      floatx4 acc = {S[dt][0] * lc.x, S[dt][1] * lc.y, S[dt][2] * lc.z, S[dt][3] * lc.w};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 kh = lds_slots_tr(KT[4], LDK, 16 * dt, s, g4, n);   // K^[kslot][16 dt + n]
        const bf16x8 kl = lds_slots_tr(KT[5], LDK, 16 * dt, s, g4, n);
        acc = mfma(kh, uh[s], acc);
        acc = mfma(kh, ul[s], acc);
        acc = mfma(kl, uh[s], acc);
      }
      S[dt] = acc;
    }
  }
  if (ST != nullptr) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<float4*>(ST + ((size_t)bh * DV + row) * DK + 16 * dt + 4 * g4) =
          make_float4(S[dt][0], S[dt][1], S[dt][2], S[dt][3]);
  }
}

// ===========================================================================
// launcher
// ===========================================================================

hipError_t launch_gated_chunked(const void* q, const void* k, const void* v,
                                const float* alpha, const float* bgate, const float* wgate,
                                const float* S0, float* ST, void* o, int B, int T, int H,
                                int dk, int dv, int out_dtype, void* workspace,
                                hipStream_t stream) {
  const int nchunks = (T + C - 1) / C;
  char* ws = static_cast<char*>(workspace);
  const dim3 pgrid(nchunks, H, B);
#define GDN_GPREP(DK_, LO_)                                                                \
  hipLaunchKernelGGL((gated_prepare_kernel<DK_, LO_>), pgrid, dim3(256), 0, stream,         \
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), alpha, bgate, \
                     ws, T, H, nchunks)
  const bool lo = out_dtype != 1;          // fp32 outputs read the lo parts of Q~ and P
  if (dk == 128) {
    if (lo) GDN_GPREP(128, true);
    else GDN_GPREP(128, false);
  } else {
    if (lo) GDN_GPREP(64, true);
    else GDN_GPREP(64, false);
  }
#undef GDN_GPREP
  const int nblocks = B * H * (dv / 64);
#define GDN_GSCAN(DK_, TO)                                                                      \
  hipLaunchKernelGGL((gated_scan_kernel<DK_, TO>), dim3(nblocks), dim3(256), 0, stream,         \
                     static_cast<const bf16*>(v), wgate, S0, static_cast<TO*>(o), ST, ws, T, H, \
                     dv, nchunks, nblocks)
  if (dk == 128) {
    if (out_dtype == 1) GDN_GSCAN(128, bf16);
    else GDN_GSCAN(128, float);
  } else {
    if (out_dtype == 1) GDN_GSCAN(64, bf16);
    else GDN_GSCAN(64, float);
  }
#undef GDN_GSCAN
  return hipGetLastError();
}

}  // namespace gdn
