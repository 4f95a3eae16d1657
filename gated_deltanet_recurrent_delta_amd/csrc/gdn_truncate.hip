// Rank-r truncation of carried states, and their stable rank.
//
// S <- U_r U_r^T S, with U_r the r leading left singular vectors of S, is the
// projection applied to every head's carried state at each 256-token segment
// boundary in "How much of its state does Gated DeltaNet use?", §3 (how
// the low-energy directions are removed; r equal to the state width leaves
// the model unchanged).  The stable rank er(S) = ||S||_F^2 / sigma_1^2 is
// "On State Reduction in Linear Attention", paper Sec. 2.2, Eq. (5).
//
// The left singular vectors of S are the eigenvectors of the symmetric
// G = S S^T (dv x dv), with eigenvalues sigma_i^2.  Method, one workgroup
// per state, in fp64 with everything in LDS:
//  1. G = S S^T from S staged in LDS 32 columns at a time.
//  2. Householder tridiagonalisation Q^T G Q = T: step k reflects row k
//     beyond the diagonal onto its first entry; the symmetric rank-2 update
//     of the trailing block runs on all threads, two barriers a step.  The
//     reflectors are packed into the rows they have freed.
//  3. The r largest eigenvalues of T by multisection: P threads per
//     eigenvalue evaluate the Sturm count (eigenvalues of T below x, from
//     the signs of the pivots of T - x I) at P points of the bracket and
//     keep the sub-interval where the count passes the eigenvalue's index.
//  4. Eigenvectors of T by one step of inverse iteration with partial
//     pivoting from a hashed start vector (the eigenvalues are exact to
//     ~1e-15 of ||T||, so one solve gives the vector); then u = Q y,
//     applying the reflectors in reverse, and a normalisation.  Vectors of
//     eigenvalues closer than 1e-6 ||T|| are made orthonormal by two passes
//     of Gram-Schmidt (any orthonormal basis of such a cluster is a valid
//     answer when it lies inside the leading r; when it straddles r the
//     leading subspace is not unique).
//  5. er = (sum of the r largest eigenvalues) / (largest), or trace / largest
//     when r >= min(dv, dk).
// This is the bisection / inverse-iteration route to selected eigenpairs
// of a symmetric matrix (Householder reduction, Sturm-sequence bisection,
// inverse iteration, back-transformation), restated for one workgroup.
// A second kernel then forms S <- U_r (U_r^T S) in fp32, 32 state columns
// per workgroup.  Only as many CUs as states are busy: the pass is bound by
// the sequential steps of 2 and 3.
#include <math.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int kEigThreads = 512;
constexpr int kEigBatch = 16;          // eigenvectors per inverse-iteration batch
constexpr int kProjCols = 32;

// One DPP move of a double (both 32-bit halves with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over aligned groups of W lanes (W a power of two, 2..64), the same
// value on every lane of a group.  Within a 16-lane row the partners come
// from DPP moves (pairs, quads, then the mirrored half row and row), across
// rows from LDS permutes.  Each step adds a lane's own partial sum to the
// other half's, as a butterfly does, so every lane of a group ends with the
// same bits.
template <int W>
__device__ __forceinline__ double lane_sum(double x) {
  if constexpr (W >= 2) x += dpp_d<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (W >= 4) x += dpp_d<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (W >= 8) x += dpp_d<0x141>(x);   // row_half_mirror
  if constexpr (W >= 16) x += dpp_d<0x140>(x);  // row_mirror
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Lane l's double (both 32-bit halves read with v_readlane; the builtin
// given a double would convert it to an integer).
__device__ __forceinline__ double readlane_d(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes, the same bits on every lane (and in every wave that
// sums the same data): 16-lane row sums by DPP, then the four row sums read
// from lanes 0, 16, 32 and 48 (no LDS permutes).
__device__ __forceinline__ double wave_sum(double x) {
  x = lane_sum<16>(x);
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}

// Minimum / maximum over the 64 lanes (same value on every lane).
__device__ __forceinline__ double wave_min(double x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmin(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ double wave_max(double x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}

// Start vector of inverse iteration: a hash of (vector, element) in
// [-0.5, 0.5), different for every vector so that the solves of a cluster
// of equal eigenvalues give independent vectors of its eigenspace.
__device__ __forceinline__ double start_value(unsigned j, unsigned i) {
  unsigned x = j * 0x9E3779B9u + i * 0x85EBCA6Bu + 0x165667B1u;
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return (double)x * 0x1p-32 - 0.5;
}

// 1 / x: v_rcp_f64 refined by two Newton steps (x finite and nonzero).
__device__ __forceinline__ double recip(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(fma(-x, r, 1.0), r, r);
  return fma(fma(-x, r, 1.0), r, r);
}

// Number of eigenvalues of the tridiagonal T (diagonal dd, squared
// off-diagonal e2) below x: the negative pivots of T - x I, q_0 = d_0 - x,
// q_i = d_i - x - e_{i-1}^2 / q_{i-1}, pivots smaller than pivmin replaced
// by -pivmin.
// The recurrence is a chain of dependent divisions; the diagonal and
// off-diagonal entries it reads (the same for every lane) are loaded from
// LDS one block of 8 steps ahead, so no step waits for them.
template <int M>
__device__ __forceinline__ int sturm_count(const double* dd, const double* e2, double x,
                                           double pivmin) {
  static_assert((M - 1) % 8 == 7, "blocks of 8 steps, the last one of 7");
  double q = dd[0] - x;
  if (fabs(q) < pivmin) q = -pivmin;
  int c = q < 0.0;
  double dn[8], en[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dn[j] = dd[1 + j];
    en[j] = e2[j];
  }
#pragma unroll 1
  for (int b = 1; b < M - 7; b += 8) {
    double dc[8], ec[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dc[j] = dn[j];
      ec[j] = en[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {               // the next block (the last has 7)
      const int i = min(b + 8 + j, M - 1);
      dn[j] = dd[i];
      en[j] = e2[i - 1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      q = fma(-ec[j], recip(q), dc[j] - x);
      if (fabs(q) < pivmin) q = -pivmin;
      c += q < 0.0;
    }
  }
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    q = fma(-en[j], recip(q), dn[j] - x);
    if (fabs(q) < pivmin) q = -pivmin;
    c += q < 0.0;
  }
  return c;
}

// Offset of reflector k in the packed store: reflector k has M - 1 - k
// entries (acting on indices k + 1 .. M - 1).
template <int M>
__device__ __forceinline__ int hv_off(int k) {
  return k * (M - 1) - k * (k - 1) / 2;
}

// M = dv, N = dk.  Grid: one block per state.  rv: eigenvectors to form (r
// when projecting, else 0); the r leading unit vectors go to U [state][K][M]
// as fp64; er[state] as described above.
template <int M, int N>
__global__ void __launch_bounds__(kEigThreads)
eig_top_kernel(const float* __restrict__ S, int r, int rv, double* __restrict__ U,
               float* __restrict__ er) {
  constexpr int K = M < N ? M : N;
  constexpr int HVSZ = M * (M - 1) / 2;      // packed reflectors
  constexpr int NB = kEigBatch;
  constexpr int SCR = 4 * NB * M;            // pivots, super, second super, rhs / y
  constexpr int BUF = HVSZ + SCR;
  constexpr int KC = 32;                     // S columns staged at a time
  static_assert((M / 32) * (M / 16) * kEigThreads == M * M, "tiles cover the matrix");
  static_assert(M * (KC + 1) <= 2 * BUF, "a staged chunk of S fits");
  static_assert((K - 1) * M <= BUF, "a cluster of K - 1 vectors fits");
  static_assert(NB * 32 == kEigThreads, "16 vectors x 32 lanes in the back-transform");

  __shared__ double buf[BUF];
  __shared__ double dd[M], ee[M], e2[M], tau[M], pv[M], lam[M], Vv[M], Wv[M], Xr[M];
  __shared__ int cl_end[M];                  // end of the cluster that starts at j (or 0)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* Sh = S + (size_t)blockIdx.x * M * N;
  double* hv = buf;                          // packed reflectors

  // ---- 1. G = S S^T, each thread's tile of it kept in registers ----------
  // tile: rows r0 .. r0 + RT - 1, columns c0 .. c0 + CT - 1; the 16 lanes of
  // a DPP row hold the 16 tiles of one block of RT rows
  // Wave wv holds row block rb (4 RT rows): waves wv and wv + 4, which
  // share a SIMD, hold blocks b and 7 - b, so that as the reduction retires
  // the leading blocks every SIMD keeps about the same work.
  constexpr int RT = M / 32, CT = M / 16;
  static_assert(kEigThreads == 512, "eight row blocks, one per wave");
  const int rb = wv < 4 ? wv : 11 - wv;
  const int r0 = RT * (4 * rb + (lane >> 4)), c0 = CT * (tid & 15);
  double A[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) A[i][j] = 0.0;
  {
    float* Sc = reinterpret_cast<float*>(buf);   // [M][KC + 1]
    for (int k0 = 0; k0 < N; k0 += KC) {
      __syncthreads();
      for (int e = tid; e < M * KC / 4; e += kEigThreads) {
        const int row = e / (KC / 4), c4 = (e - row * (KC / 4)) * 4;
        const float4 v = *reinterpret_cast<const float4*>(Sh + (size_t)row * N + k0 + c4);
        float* d = Sc + row * (KC + 1) + c4;
        d[0] = v.x;
        d[1] = v.y;
        d[2] = v.z;
        d[3] = v.w;
      }
      __syncthreads();
#pragma unroll 4
      for (int kk = 0; kk < KC; ++kk) {
        double a[RT], b[CT];
#pragma unroll
        for (int i = 0; i < RT; ++i) a[i] = Sc[(r0 + i) * (KC + 1) + kk];
#pragma unroll
        for (int j = 0; j < CT; ++j) b[j] = Sc[(c0 + j) * (KC + 1) + kk];
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int j = 0; j < CT; ++j) A[i][j] = fma(a[i], b[j], A[i][j]);
      }
    }
  }
  if (r0 == 0) {
#pragma unroll
    for (int j = 0; j < CT; ++j) Xr[c0 + j] = A[0][j];
  }
  __syncthreads();                                 // row 0 in Xr; the staging is free

  // ---- 2. Householder tridiagonalisation ----------------------------------
  // Step k: x = row k beyond the diagonal (in Xr), v = x - alpha e_1 (zero
  // at indices <= k), p = t A v, w = p - (t/2)(p.v) v, A -= v w^T + w v^T
  // on the whole matrix: the full similarity H A H, which leaves row and
  // column k as (d_k, alpha) and needs no masks.  v and w sit in LDS (Vv,
  // Wv); every wave computes and writes them itself (bitwise the same
  // values), so they need no barrier of their own.  Row k + 1 goes to Xr
  // for the next step.
  // A wave whose rows are all <= k has nothing left to do: its rows are
  // final (v and w vanish there) and no later step reads them, so it only
  // passes the barriers; the wave with the last block (always active)
  // records the tridiagonal entries and the reflectors.
  constexpr int EL = (M + 63) / 64;                // entries of a row per lane
  const bool last_block = rb == 7;
  for (int k = 0; k < M - 2; ++k) {
    if (4 * RT * rb + 4 * RT - 1 <= k) {
      __syncthreads();
      __syncthreads();
      continue;
    }
    double xl[EL];
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int j = lane + 64 * e;
      xl[e] = (j > k && j < M) ? Xr[j] : 0.0;
      s = fma(xl[e], xl[e], s);
    }
    s = wave_sum(s);
    const double x0 = Xr[k + 1];
    double alpha = 0.0, t = 0.0, v0 = 0.0;
    if (s > 0.0) {
      const double nx = sqrt(s);
      alpha = -copysign(nx, x0);
      v0 = x0 - alpha;
      t = 1.0 / (nx * (nx + fabs(x0)));            // 2 / v^T v
    }
    if (last_block && lane == 0) {
      dd[k] = Xr[k];
      ee[k] = alpha;
      tau[k] = t;
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int j = lane + 64 * e;
      const double vj = j == k + 1 ? v0 : xl[e];
      if (j < M) Vv[j] = vj;
      if (last_block && j > k && j < M) hv[hv_off<M>(k) + j - k - 1] = vj;
    }
    // p = t A v
    double vc[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) vc[j] = Vv[c0 + j];
    double pr[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < CT; ++j) acc = fma(A[i][j], vc[j], acc);
      pr[i] = lane_sum<16>(acc);
    }
    if ((tid & 15) == 0) {
#pragma unroll
      for (int i = 0; i < RT; ++i) pv[r0 + i] = t * pr[i];
    }
    __syncthreads();
    // w = p - (t/2) (p . v) v
    double kl = 0.0;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int j = lane + 64 * e;
      if (j < M) kl = fma(pv[j], Vv[j], kl);
    }
    const double kv = 0.5 * t * wave_sum(kl);
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int j = lane + 64 * e;
      if (j < M) Wv[j] = pv[j] - kv * Vv[j];
    }
    // A -= v w^T + w v^T
    double wc[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) wc[j] = Wv[c0 + j];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const double vi = Vv[r0 + i], wi = Wv[r0 + i];
#pragma unroll
      for (int j = 0; j < CT; ++j) A[i][j] = fma(-vi, wc[j], fma(-wi, vc[j], A[i][j]));
    }
    // row k + 1 for the next step (Xr was last read before the barrier)
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      if (r0 + i == k + 1) {
#pragma unroll
        for (int j = 0; j < CT; ++j) Xr[c0 + j] = A[i][j];
      }
    }
    __syncthreads();
  }
  // the trailing 2 x 2 block: row M - 2 is in Xr, A[M-1][M-1] with its owner
  if (tid == 0) {
    dd[M - 2] = Xr[M - 2];
    ee[M - 2] = Xr[M - 1];
    ee[M - 1] = 0.0;
  }
  if (r0 + RT - 1 == M - 1 && c0 + CT - 1 == M - 1) dd[M - 1] = A[RT - 1][CT - 1];
  __syncthreads();
  if (tid < M) e2[tid] = ee[tid] * ee[tid];

  // ---- 3. the nl largest eigenvalues -------------------------------------
  double lo = HUGE_VAL, hi = -HUGE_VAL, emax = 0.0;
  for (int i = lane; i < M; i += 64) {
    const double ea = i > 0 ? fabs(ee[i - 1]) : 0.0, eb = fabs(ee[i]);
    lo = fmin(lo, dd[i] - ea - eb);
    hi = fmax(hi, dd[i] + ea + eb);
    emax = fmax(emax, eb * eb);
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  emax = wave_max(emax);
  const double tnorm = fmax(fabs(lo), fabs(hi));
  const double pivmin = 0x1p-1022 * fmax(1.0, emax);
  lo -= 0x1p-46 * tnorm + pivmin;
  hi += 0x1p-46 * tnorm + pivmin;
  const bool zero = !(tnorm > 0.0);
  const int nl = rv > 0 ? rv : 1;                 // eigenvalues to locate
  // P threads per eigenvalue and the multisection steps for ~50 bits.  The
  // counts are chains of fp64 divisions: with one wave per SIMD each chain
  // runs at its latency, with two the SIMD's fp64 issue rate is the limit
  // and costs more than the extra steps of a smaller P, so nl * P stays
  // within 256 threads (measured on MI355X, 16 heads of 128 x 128: r = 12
  // 417 -> 395 us, r = 32 516 -> 486 us per boundary).
  const int P = nl <= 4 ? 64 : nl <= 8 ? 32 : nl <= 16 ? 16 : nl <= 32 ? 8 : nl <= 64 ? 4 : 2;
  const int nit = P == 64 ? 9 : P == 32 ? 10 : P == 16 ? 13 : P == 8 ? 16 : P == 4 ? 22 : 32;
  __syncthreads();                                 // e2 complete
  {
    const int j = tid / P, p = tid - j * P;
    if (j < nl) {
      double a = lo, b = hi;
      const int target = M - j;                    // count(x) >= M - j  <=>  x > lambda_j
      const int gbase = (tid & 63) - p;            // first lane of the group in the wave
      const uint64_t gmask = P == 64 ? ~0ull : ((1ull << P) - 1);
      for (int it = 0; it < nit; ++it) {
        const double w = (b - a) / (P + 1);
        const int c = sturm_count<M>(dd, e2, a + w * (p + 1), pivmin);
        const uint64_t hit = (__ballot(c >= target) >> gbase) & gmask;
        if (hit == 0) {
          a = a + w * P;
        } else {
          const int ps = __builtin_ctzll(hit);
          const double nb = a + w * (ps + 1);
          if (ps > 0) a = a + w * ps;
          b = nb;
        }
      }
      if (p == 0) lam[j] = 0.5 * (a + b);
    }
  }
  __syncthreads();

  // ---- 4. eigenvectors ------------------------------------------------------
  if (rv > 0) {
    double* sd = buf + HVSZ;                       // element (i, t) at i * NB + t; 1 / pivot
    double* ss = sd + NB * M;
    double* s2 = ss + NB * M;
    double* sy = s2 + NB * M;
    double* Uh = U + (size_t)blockIdx.x * K * M;
    for (int jb = 0; jb < rv; jb += NB) {
      const int nbv = min(NB, rv - jb);
      if (tid < nbv && !zero) {
        // (T - lambda I) y = x by Gaussian elimination with partial pivoting;
        // row i of the reduced system is [pivot, super, second super], kept
        // as [1 / pivot, super, second super]
        const int t = tid, j = jb + t;
        const double lj = lam[j], tiny = 0x1p-52 * tnorm;
        double a_cur = dd[0] - lj, b_cur = ee[0], y_cur = start_value(j, 0);
        for (int i = 0; i < M - 1; ++i) {
          const double sub = ee[i], a_nx = dd[i + 1] - lj, b_nx = ee[i + 1];
          const double y_nx = start_value(j, i + 1);
          // both cases by selects (one reciprocal, no divergent branch)
          const bool sw = fabs(a_cur) < fabs(sub);         // rows i and i + 1 swap
          const double piv = recip(sw ? sub : (a_cur != 0.0 ? a_cur : tiny));
          const double mlt = (sw ? a_cur : sub) * piv;
          sd[i * NB + t] = piv;
          ss[i * NB + t] = sw ? a_nx : b_cur;
          s2[i * NB + t] = sw ? b_nx : 0.0;
          sy[i * NB + t] = sw ? y_nx : y_cur;
          const double an = sw ? fma(-mlt, a_nx, b_cur) : fma(-mlt, b_cur, a_nx);
          const double bn = sw ? -mlt * b_nx : b_nx;
          const double yn = sw ? fma(-mlt, y_nx, y_cur) : fma(-mlt, y_cur, y_nx);
          a_cur = an;
          b_cur = bn;
          y_cur = yn;
        }
        sd[(M - 1) * NB + t] = recip(a_cur != 0.0 ? a_cur : tiny);
        ss[(M - 1) * NB + t] = 0.0;
        s2[(M - 1) * NB + t] = 0.0;
        sy[(M - 1) * NB + t] = y_cur;
        double y1 = 0.0, y2 = 0.0;                 // y_{i+1}, y_{i+2}
#pragma unroll 8
        for (int i = M - 1; i >= 0; --i) {
          const double yi =
              (sy[i * NB + t] - ss[i * NB + t] * y1 - s2[i * NB + t] * y2) * sd[i * NB + t];
          sy[i * NB + t] = yi;
          y2 = y1;
          y1 = yi;
        }
      }
      __syncthreads();
      {
        // u = H_0 H_1 ... H_{M-3} y, normalised: one 16-lane DPP row per
        // vector (the dot products need no cross-row step), 8 entries a lane
        constexpr int EPL = M / 16;
        const int t = tid >> 4, l = tid & 15;
        double u[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          u[e] = (t < nbv && !zero) ? sy[(l + 16 * e) * NB + t] : 0.0;
        if (t < NB) {
#pragma unroll 2
          for (int k = M - 3; k >= 0; --k) {
            const double* vk = hv + hv_off<M>(k) - (k + 1);   // vk[i] for i > k
            double vv[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const int i = l + 16 * e;
              vv[e] = i > k ? vk[i] : 0.0;
            }
            double d0 = 0.0, d1 = 0.0;
#pragma unroll
            for (int e = 0; e < EPL; e += 2) {
              d0 = fma(u[e], vv[e], d0);
              d1 = fma(u[e + 1], vv[e + 1], d1);
            }
            const double dot = lane_sum<16>(d0 + d1) * tau[k];
#pragma unroll
            for (int e = 0; e < EPL; ++e) u[e] = fma(-dot, vv[e], u[e]);
          }
        }
        double nn = 0.0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) nn = fma(u[e], u[e], nn);
        nn = lane_sum<16>(nn);
        const double sc = nn > 0.0 ? 1.0 / sqrt(nn) : 0.0;
        if (t < nbv) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) Uh[(size_t)(jb + t) * M + l + 16 * e] = u[e] * sc;
        }
      }
      __syncthreads();
    }

    // clusters: consecutive eigenvalues closer than 1e-6 ||T||
    if (tid == 0) {
      const double ctol = 1e-6 * tnorm;
      int c0 = 0;
      for (int j = 1; j <= rv; ++j) {
        if (j == rv || lam[j - 1] - lam[j] > ctol) {
          cl_end[c0] = j;
          for (int q = c0 + 1; q < j; ++q) cl_end[q] = 0;
          c0 = j;
        }
      }
    }
    __syncthreads();
    if (!zero) {
      for (int c0 = 0; c0 < rv;) {
        const int c1 = cl_end[c0], n = c1 - c0;
        if (n >= 2) {
          // two passes of classical Gram-Schmidt per vector, in LDS
          double* W = buf;
          for (int e = tid; e < n * M; e += kEigThreads) W[e] = Uh[(size_t)c0 * M + e];
          __syncthreads();
          for (int a = 1; a < n; ++a) {
            for (int pass = 0; pass < 2; ++pass) {
              for (int b = wv; b < a; b += kEigThreads / 64) {
                double d = 0.0;
                for (int i = lane; i < M; i += 64) d = fma(W[a * M + i], W[b * M + i], d);
                d = wave_sum(d);
                if (lane == 0) pv[b] = d;
              }
              __syncthreads();
              if (tid < M) {
                double x = W[a * M + tid];
                for (int b = 0; b < a; ++b) x = fma(-pv[b], W[b * M + tid], x);
                W[a * M + tid] = x;
              }
              __syncthreads();
            }
            if (wv == 0) {
              double d = 0.0;
              for (int i = lane; i < M; i += 64) d = fma(W[a * M + i], W[a * M + i], d);
              d = wave_sum(d);
              if (lane == 0) pv[0] = d > 0.0 ? 1.0 / sqrt(d) : 0.0;
            }
            __syncthreads();
            if (tid < M) W[a * M + tid] *= pv[0];
            __syncthreads();
          }
          for (int e = tid; e < n * M; e += kEigThreads) Uh[(size_t)c0 * M + e] = W[e];
          __syncthreads();
        }
        c0 = c1;
      }
    }
  }

  // ---- 5. stable rank -----------------------------------------------------
  if (er != nullptr && tid == 0) {
    float res = __builtin_nanf("");
    if (!zero && lam[0] > 0.0) {
      double tot = 0.0;
      if (rv > 0) {
        for (int j = 0; j < rv; ++j) tot += lam[j];
      } else {
        for (int i = 0; i < M; ++i) tot += dd[i];
      }
      res = (float)(tot / lam[0]);
    }
    er[blockIdx.x] = res;
  }
}

// S <- U_r (U_r^T S) for kProjCols state columns of one head.
// Grid: (N / kProjCols, heads).
template <int M, int N>
__global__ void __launch_bounds__(256)
project_kernel(float* __restrict__ S, int r, const double* __restrict__ U) {
  constexpr int K = M < N ? M : N;
  constexpr int CB = kProjCols;
  __shared__ float Us[(K - 1) * M];          // r <= K - 1 unit vectors
  __shared__ float Sb[M][CB + 1];
  __shared__ float W[K - 1][CB + 1];

  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * CB;
  float* Sh = S + (size_t)blockIdx.y * M * N;
  const double* Uh = U + (size_t)blockIdx.y * K * M;
  for (int e = tid; e < r * M; e += 256) Us[e] = (float)Uh[e];
  for (int e = tid; e < M * CB; e += 256) {
    const int i = e / CB, c = e % CB;
    Sb[i][c] = Sh[(size_t)i * N + c0 + c];
  }
  __syncthreads();
  for (int e = tid; e < r * CB; e += 256) {
    const int j = e / CB, c = e % CB;
    float acc = 0.0f;
#pragma unroll 8
    for (int i = 0; i < M; ++i) acc += Us[j * M + i] * Sb[i][c];
    W[j][c] = acc;
  }
  __syncthreads();
  for (int e = tid; e < M * CB; e += 256) {
    const int i = e / CB, c = e % CB;
    float acc = 0.0f;
    for (int j = 0; j < r; ++j) acc += Us[j * M + i] * W[j][c];
    Sh[(size_t)i * N + c0 + c] = acc;
  }
}

template <int M, int N>
hipError_t launch_truncate_t(float* S, int BH, int r, float* er, double* U,
                             hipStream_t stream) {
  constexpr int K = M < N ? M : N;
  const bool project = r < K;
  if (project || er != nullptr) {
    hipLaunchKernelGGL((eig_top_kernel<M, N>), dim3(BH), dim3(kEigThreads), 0, stream, S,
                       r, project ? r : 0, project ? U : nullptr, er);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (project) {
    hipLaunchKernelGGL((project_kernel<M, N>), dim3(N / kProjCols, BH),
                       dim3(256), 0, stream, S, r, U);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_truncate(float* S, int BH, int dv, int dk, int r, float* er,
                           double* U, hipStream_t stream) {
  if (dv == 128 && dk == 128) return launch_truncate_t<128, 128>(S, BH, r, er, U, stream);
  if (dv == 128 && dk == 64) return launch_truncate_t<128, 64>(S, BH, r, er, U, stream);
  if (dv == 64 && dk == 128) return launch_truncate_t<64, 128>(S, BH, r, er, U, stream);
  return launch_truncate_t<64, 64>(S, BH, r, er, U, stream);
}

}  // namespace gdn
