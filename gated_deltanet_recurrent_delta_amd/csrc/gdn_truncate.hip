// Rank-r truncation of carried states, and their stable rank.
//
// S <- U_r U_r^T S, with U_r the r leading left singular vectors of S, is the
// projection applied to every head's carried state at each 256-token segment
// boundary in "How much of its state does Gated DeltaNet use?", §3 (how
// the low-energy directions are removed; r equal to the state width leaves
// the model unchanged).  The stable rank er(S) = ||S||_F^2 / sigma_1^2 is
// "On State Reduction in Linear Attention", paper Sec. 2.2, Eq. (5).
//
// Method, one workgroup per head, everything in fp64 in LDS:
//  1. Householder QR of X = S^T (dk x dv, no pivoting).  S^T = Q R gives
//     S = R^T Q^T, so the left singular vectors of S are those of L = R^T;
//     Q is never formed.
//  2. One-sided (Hestenes) Jacobi on the K = min(dv, dk) columns of L (the
//     rows of R), pairs taken in round-robin order so that each round's K/2
//     rotations touch disjoint columns and run in parallel.  At convergence
//     L V = U Sigma: column j is sigma_j u_j, so V is never formed either.
//     Starting from R instead of S roughly halves the sweeps on the states'
//     decaying spectra (the QR-preconditioned Jacobi SVD of Drmac and
//     Veselic).
//  3. The column norms are ranked; the r leading unit columns go to the
//     workspace as fp32 and er = (sum of the r largest sigma^2) / sigma_1^2.
// A second kernel then forms S <- U_r (U_r^T S) in fp32, 32 state columns per
// workgroup.  The workload (16 heads at a time) is latency bound: it fills
// only as many CUs as there are heads.
#include <math.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {
namespace {

constexpr int kSvdThreads = 512;
constexpr int kMaxSweeps = 30;
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

// M = dv (length of a state column), N = dk.  Grid: one block per head.
template <int M, int N>
__global__ void __launch_bounds__(kSvdThreads)
svd_left_kernel(const float* __restrict__ S, int r, float* __restrict__ U,
                float* __restrict__ er) {
  constexpr int K = M < N ? M : N;           // rows of R = columns of L
  constexpr int NSTEP = (N - 1 < M) ? N - 1 : M;   // Householder steps
  constexpr int LD = M + 8;                  // X row stride (doubles)
  constexpr int G = kSvdThreads / M;         // row groups in the QR update
  constexpr int NP = K / 2;                  // rotations per round
  constexpr int TPP = kSvdThreads / NP;      // lanes per rotation
  constexpr int RPT = M / TPP;               // elements per lane per column
  static_assert(TPP <= 64 && RPT * TPP == M && G * M == kSvdThreads, "");

  __shared__ double X[N * LD];               // X[j][c] = S[c][j]
  __shared__ double vec[N];
  __shared__ double part[G][M];
  __shared__ double red[kSvdThreads / 64];
  __shared__ double nrm[K];
  __shared__ int rank_s[K];
  __shared__ double tau_s;

  const int tid = threadIdx.x;
  const float* Sh = S + (size_t)blockIdx.x * M * N;

  // ---- load X = S^T and ||S||_F^2
  double fro = 0.0;
#pragma unroll 4
  for (int e = tid; e < M * N; e += kSvdThreads) {
    const double x = Sh[e];
    X[(e % N) * LD + e / N] = x;
    fro += x * x;
  }
  fro = lane_sum<64>(fro);
  if ((tid & 63) == 0) red[tid >> 6] = fro;
  __syncthreads();
  fro = 0.0;
  for (int w = 0; w < kSvdThreads / 64; ++w) fro += red[w];

  // ---- Householder QR: step k zeroes column k below the diagonal
  const int cc = tid % M, g = tid / M;
  for (int k = 0; k < NSTEP; ++k) {
    if (tid < 64) {
      double s = 0.0;
      for (int j = k + 1 + tid; j < N; j += 64) {
        const double x = X[j * LD + k];
        s += x * x;
      }
      s = lane_sum<64>(s);
      const double x0 = X[k * LD + k];
      double tau = 0.0, v0 = 1.0, diag = x0;
      if (s > 0.0) {
        const double nx = sqrt(x0 * x0 + s);
        diag = x0 >= 0.0 ? -nx : nx;          // reflect away from x0's sign
        v0 = x0 - diag;
        tau = 2.0 / (v0 * v0 + s);
      }
      for (int j = k + tid; j < N; j += 64)
        vec[j] = j == k ? v0 : X[j * LD + k];
      if (tid == 0) tau_s = tau;
      __builtin_amdgcn_wave_barrier();
      if (tid == 0) X[k * LD + k] = diag;
    }
    __syncthreads();
    const double tau = tau_s;
    double p = 0.0;
    if (cc > k) {
#pragma unroll 4
      for (int j = k + g; j < N; j += G) p += vec[j] * X[j * LD + cc];
    }
    part[g][cc] = p;
    __syncthreads();
    if (cc > k && tau != 0.0) {
      double w = 0.0;
#pragma unroll
      for (int h = 0; h < G; ++h) w += part[h][cc];
      w *= tau;
#pragma unroll 4
      for (int j = k + g; j < N; j += G) X[j * LD + cc] -= vec[j] * w;
    }
    __syncthreads();
  }
  // R is the upper trapezoid of the first K rows; clear what lies below it
#pragma unroll 1
  for (int e = tid; e < K * M; e += kSvdThreads) {
    const int j = e / M, c = e % M;
    if (c < j) X[j * LD + c] = 0.0;
  }
  __syncthreads();

  // ---- one-sided Jacobi on the rows 0..K-1 of X (the columns of L)
  const int pair = tid / TPP, sub = tid % TPP;
  const double tol = M * 0x1p-53;            // |cos| below this: orthogonal
  const double negl = tol * tol * fro;       // columns this small are zero
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    int rotated = 0;
#pragma unroll 1
    for (int rnd = 0; rnd < K - 1; ++rnd) {
      // round-robin pairing: column K-1 stays, the others rotate
      int p = rnd, q = K - 1;
      if (pair != 0) {
        p = rnd + pair;
        if (p >= K - 1) p -= K - 1;
        q = rnd - pair;
        if (q < 0) q += K - 1;
      }
      double* xp = X + p * LD;
      double* xq = X + q * LD;
      double a[RPT], b[RPT];
      double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll
      for (int j = 0; j < RPT; ++j) {
        a[j] = xp[sub + j * TPP];
        b[j] = xq[sub + j * TPP];
        al += a[j] * a[j];
        be += b[j] * b[j];
        ga += a[j] * b[j];
      }
      al = lane_sum<TPP>(al);
      be = lane_sum<TPP>(be);
      ga = lane_sum<TPP>(ga);
      // every lane of the group holds the same sums (the butterfly adds the
      // same two values in both orders), so they all take the same branch
      if (fmin(al, be) > negl && fabs(ga) > tol * sqrt(al) * sqrt(be)) {
        // tan of the angle that makes the pair orthogonal: the smaller root
        // of t^2 + 2 zeta t - 1 = 0
        const double zeta = (be - al) / (2.0 * ga);
        const double t = fabs(zeta) > 1e100
                             ? 0.5 / zeta
                             : copysign(1.0, zeta) /
                                   (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double cs = 1.0 / sqrt(1.0 + t * t);
        const double sn = cs * t;
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
          xp[sub + j * TPP] = cs * a[j] - sn * b[j];
          xq[sub + j * TPP] = sn * a[j] + cs * b[j];
        }
        rotated = 1;
      }
      __syncthreads();
    }
    if (!__syncthreads_or(rotated)) break;
  }

  // ---- sigma_j^2 = ||column j||^2, ranks, stable rank, unit columns
  {
    const int j0 = 2 * pair, j1 = j0 + 1;
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const double x0 = X[j0 * LD + sub + j * TPP];
      const double x1 = X[j1 * LD + sub + j * TPP];
      s0 += x0 * x0;
      s1 += x1 * x1;
    }
    s0 = lane_sum<TPP>(s0);
    s1 = lane_sum<TPP>(s1);
    if (sub == 0) {
      nrm[j0] = s0;
      nrm[j1] = s1;
    }
  }
  __syncthreads();
  // (loops over the K norms are kept rolled: unrolled, the K doubles would
  // all be held in registers)
  double smax = 0.0;
#pragma unroll 4
  for (int j = 0; j < K; ++j) smax = fmax(smax, nrm[j]);
  if (tid < K) {
    const double me = nrm[tid];
    int cnt = 0;
#pragma unroll 4
    for (int j = 0; j < K; ++j) {
      const double o = nrm[j];
      cnt += (o > me) || (o == me && j < tid);
    }
    rank_s[tid] = cnt;
  }
  __syncthreads();
  if (er != nullptr && tid == 0) {
    double tot = 0.0;
#pragma unroll 4
    for (int j = 0; j < K; ++j)
      if (rank_s[j] < r) tot += nrm[j];
    er[blockIdx.x] = smax > 0.0 ? (float)(tot / smax) : __builtin_nanf("");
  }
  if (U != nullptr && r < K) {
    // a column below 2^-50 sigma_1 carries no direction worth keeping
    const double floor = smax * 0x1p-100;
    float* Uh = U + (size_t)blockIdx.x * K * M;
#pragma unroll 1
    for (int e = tid; e < K * M; e += kSvdThreads) {
      const int j = e / M, c = e % M;
      const int rk = rank_s[j];
      if (rk < r) {
        const double n2 = nrm[j];
        Uh[rk * M + c] = n2 > floor ? (float)(X[j * LD + c] / sqrt(n2)) : 0.0f;
      }
    }
  }
}

// S <- U_r (U_r^T S) for kProjCols state columns of one head.
// Grid: (N / kProjCols, heads).
template <int M, int N>
__global__ void __launch_bounds__(256)
project_kernel(float* __restrict__ S, int r, const float* __restrict__ U) {
  constexpr int K = M < N ? M : N;
  constexpr int CB = kProjCols;
  __shared__ float Us[(K - 1) * M];          // r <= K - 1 unit vectors
  __shared__ float Sb[M][CB + 1];
  __shared__ float W[K - 1][CB + 1];

  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * CB;
  float* Sh = S + (size_t)blockIdx.y * M * N;
  const float* Uh = U + (size_t)blockIdx.y * K * M;
  for (int e = tid; e < r * M; e += 256) Us[e] = Uh[e];
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
hipError_t launch_truncate_t(float* S, int BH, int r, float* er, float* U,
                             hipStream_t stream) {
  constexpr int K = M < N ? M : N;
  const bool project = r < K;
  if (project || er != nullptr) {
    hipLaunchKernelGGL((svd_left_kernel<M, N>), dim3(BH), dim3(kSvdThreads),
                       0, stream, S, r, project ? U : nullptr, er);
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
                           float* U, hipStream_t stream) {
  if (dv == 128 && dk == 128) return launch_truncate_t<128, 128>(S, BH, r, er, U, stream);
  if (dv == 128 && dk == 64) return launch_truncate_t<128, 64>(S, BH, r, er, U, stream);
  if (dv == 64 && dk == 128) return launch_truncate_t<64, 128>(S, BH, r, er, U, stream);
  return launch_truncate_t<64, 64>(S, BH, r, er, U, stream);
}

}  // namespace gdn
