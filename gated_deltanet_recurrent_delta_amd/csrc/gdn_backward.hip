// Backward pass of the gated delta rule, recurrent form, on gfx950.
//
// The forward step (per head and token; "On State Reduction in Linear
// Attention" reading notes, paper Sec. 2.1 with the per-token scalar decay, and
// "Linear Attention Architectures" reading notes, paper Sec. 3.3 for the order
// decay -> predict -> write -> read):
//     S~ = alpha S_prev,  w = v - S~ k,  u = beta w,  S = S~ + u k^T,  o = S q
// The pages train these layers but print no backward pass; this is the
// derivative of that step.  With G the gradient reaching S (dS from the
// later tokens plus do q^T):
//     dq = S^T do          du = G k              dv = beta du
//     dk = G^T u - beta S~^T du                  dbeta = du . w
//     dS~ = G - beta du k^T                      dalpha = <dS~, S_prev>
//     dS_prev = alpha dS~
// Per state row s_i (value channel i) the forward step and the backward step
// of row i of G only touch row i, so rows run independently as in the
// forward recurrent kernel: 16 lanes per row, dk/64 float4 per lane, 4 NG
// rows per wave.  dv is per row; dq, dk, dalpha and dbeta are sums over the
// dv rows of a head.
//
// The backward step needs S_prev, which the forward step does not let one
// recover (I - beta k k^T is singular at beta |k|^2 = 1), so:
//   1. each wave first runs its rows forward over the sequence and stores
//      the state every L tokens (checkpoints in the workspace);
//   2. then, block by block from the end, it reruns the L tokens of a block
//      from its checkpoint with the L states in registers and steps back
//      through them.
// The sums over rows: shuffles over the 4 rows of a wave, then LDS over the
// 4 waves of the workgroup (one barrier per block of L tokens), then one
// partial per workgroup and token in the workspace, which a second kernel
// adds up over the workgroups of the head.  Every sum is taken in a fixed
// order, so the results do not depend on timing.  This is the first correct
// form: the chunked form, with the products on MFMA, is the faster one.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kBwdL = 8;          // tokens between state checkpoints
constexpr int kBwdWaves = 4;      // waves per workgroup

template <int F>
__device__ __forceinline__ float dot4(const floatx4 (&a)[F], const float4 (&b)[F]) {
  float p = 0.f;
#pragma unroll
  for (int f = 0; f < F; ++f) p += a[f][0] * b[f].x + a[f][1] * b[f].y + a[f][2] * b[f].z + a[f][3] * b[f].w;
  return p;
}

// Inputs kept as loaded (bf16 bits, or fp32) until they are used, so that a
// block's loads can be issued ahead of other work without the conversions
// (which wait for the data) coming with them.
__device__ __forceinline__ uint2 ld_raw4(const bf16* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ float4 ld_raw4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 cvt4(uint2 u) {
  return make_float4(bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16),
                     bf16_bits_to_f32(u.y & 0xFFFFu), bf16_bits_to_f32(u.y >> 16));
}
__device__ __forceinline__ float4 cvt4(float4 x) { return x; }
__device__ __forceinline__ uint16_t ld_raw1(const bf16* p) { return *reinterpret_cast<const uint16_t*>(p); }
__device__ __forceinline__ float ld_raw1(const float* p) { return *p; }
__device__ __forceinline__ float cvt1(uint16_t u) { return bf16_bits_to_f32(u); }
__device__ __forceinline__ float cvt1(float x) { return x; }

__device__ __forceinline__ float xsum_rows(float x) {   // over lanes l, l^16, l^32, l^48
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

}  // namespace

// 8 rows per wave at either key width: at dk = 128 that is 254 registers and
// two waves per SIMD, and the workgroups of a B=8, H=16 batch (512) are all
// resident at once (4 rows per wave: 157 registers, 1024 workgroups in two
// rounds, 21.1 ms against 15.0 ms at B=8, T=4096, H=16).
int backward_ng(int) { return 2; }

// Workgroups per head and the width of one partial (dq, dk, dalpha, dbeta).
int backward_wgs(int dk, int dv) { return dv / (4 * backward_ng(dk) * kBwdWaves); }
int backward_pw(int dk) { return 2 * dk + 2; }

size_t backward_ws_floats(int B, int T, int H, int dk, int dv, size_t* ckpt_floats) {
  const size_t BH = (size_t)B * H;
  const size_t nc = ((size_t)T + kBwdL - 1) / kBwdL;
  const size_t ck = BH * nc * dv * dk;
  const size_t ckr = (ck + 63) / 64 * 64;               // partials 256-byte aligned
  if (ckpt_floats) *ckpt_floats = ckr;
  return ckr + BH * (size_t)T * backward_wgs(dk, dv) * backward_pw(dk);
}

template <int DK, int NG, typename TIn>
__global__ __launch_bounds__(64 * kBwdWaves) void backward_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* S0,
    const TIn* __restrict__ dO, const float* dST, float* __restrict__ dv_out, float* dS0,
    float* __restrict__ ckpt, float* __restrict__ part, int H, int T, int dv) {
  constexpr int F = DK / 64;
  constexpr int L = kBwdL;
  constexpr int PW = 2 * DK + 2;          // partial: dq, dk, dalpha, dbeta
  constexpr int PWS = 2 * DK + 4;         // its LDS stride (16-byte rows)
  constexpr int ROWS_WG = 4 * NG * kBwdWaves;
  __shared__ __attribute__((aligned(16))) float red[L][kBwdWaves][PWS];
  // dalpha (lanes 0..31) and dbeta (lanes 32..63): a slot per lane, so the
  // store needs no branch (which would end the scheduling region per token)
  __shared__ float red2[L][kBwdWaves][64];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wgs = dv / ROWS_WG;                         // grid = B H wgs exactly
  const int head = blockIdx.x / wgs;
  const int wg = blockIdx.x - head * wgs;
  const int row0 = wg * ROWS_WG + wv * 4 * NG + (lane >> 4);   // rows row0 + 4 g
  const int sub = lane & 15;
  const int b = head / H, h = head - b * H;
  const int nc = (T + L - 1) / L;

  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };
  auto srow = [&](int g) { return ((size_t)head * dv + row0 + 4 * g) * DK; };
  auto crow = [&](int c, int g) {
    return (((size_t)head * nc + c) * dv + row0 + 4 * g) * DK;
  };
  // Token inputs.  Every load is unconditional, from a clamped token index,
  // and a token past the end gets the identity gates (alpha 1, beta 0, no
  // output gradient): the loops over a block then have no branch, and the
  // compiler is free to issue a block's loads ahead of its dependent chain.
  using RawK = decltype(ld_raw4(k));
  using RawV = decltype(ld_raw1(v));
  struct Tok {
    RawK k[F];
    float a, be;
    RawV v[NG];
  };
  auto load_tok = [&](Tok& x, int t) {
    const size_t ti = tok(min(t, T - 1));
    const bool ok = t < T;
#pragma unroll
    for (int f = 0; f < F; ++f) x.k[f] = ld_raw4(k + ti * DK + 64 * f + 4 * sub);
    // loaded unconditionally, then selected: a load under the condition
    // becomes a branch, which ends the scheduling region at every token
    const float a = alpha[ti], be = beta[ti];
    x.a = ok ? a : 1.f;
    x.be = ok ? be : 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) x.v[g] = ld_raw1(v + ti * dv + row0 + 4 * g);
  };
  // one forward step of the NG rows held in s
  auto fwd = [&](const floatx4 (&s)[NG][F], floatx4 (&out)[NG][F], const Tok& x) {
    float4 kk[F];
#pragma unroll
    for (int f = 0; f < F; ++f) kk[f] = cvt4(x.k[f]);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      floatx4 sa[F];
#pragma unroll
      for (int f = 0; f < F; ++f) sa[f] = s[g][f] * x.a;
      const float u = x.be * (cvt1(x.v[g]) - sum16(dot4<F>(sa, kk)));
#pragma unroll
      for (int f = 0; f < F; ++f)
        out[g][f] = floatx4{sa[f][0] + u * kk[f].x, sa[f][1] + u * kk[f].y,
                            sa[f][2] + u * kk[f].z, sa[f][3] + u * kk[f].w};
    }
  };

  // 1. forward over the sequence, a checkpoint before every L-th token
  {
    floatx4 s[NG][F];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int f = 0; f < F; ++f)
        s[g][f] = S0 ? *reinterpret_cast<const floatx4*>(S0 + srow(g) + 64 * f + 4 * sub)
                     : floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nc; ++c) {
      // the block's loads go out before the checkpoint stores: stores count
      // in the same in-order counter as loads, so a wait for a load issued
      // after them would also wait for the stores
      Tok xs[L];
#pragma unroll
      for (int i = 0; i < L; ++i) load_tok(xs[i], c * L + i);
      __builtin_amdgcn_sched_barrier(0);      // keep them there
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int f = 0; f < F; ++f)
          *reinterpret_cast<floatx4*>(ckpt + crow(c, g) + 64 * f + 4 * sub) = s[g][f];
#pragma unroll
      for (int i = 0; i < L; ++i) fwd(s, s, xs[i]);
    }
  }

  // 2. backward, block by block from the end
  floatx4 G[NG][F];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int f = 0; f < F; ++f)
      G[g][f] = dST ? *reinterpret_cast<const floatx4*>(dST + srow(g) + 64 * f + 4 * sub)
                    : floatx4{0.f, 0.f, 0.f, 0.f};
  // A block's checkpoint and the inputs of its rerun are loaded before the
  // previous block's stores (the loop carries them), for the same reason as
  // in the forward pass; the block's states are dead by then, so they fit.
  floatx4 stn[NG][F];
  Tok xn[L - 1];
  auto prefetch = [&](int c) {                          // block c (clamped to 0)
    const int cc = max(c, 0);
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int f = 0; f < F; ++f)
        stn[g][f] = *reinterpret_cast<const floatx4*>(ckpt + crow(cc, g) + 64 * f + 4 * sub);
#pragma unroll
    for (int i = 0; i + 1 < L; ++i) load_tok(xn[i], cc * L + i);
  };
  if (nc > 0) prefetch(nc - 1);
  for (int c = nc - 1; c >= 0; --c) {
    const int t0 = c * L, n = min(L, T - t0);           // uniform in the workgroup
    floatx4 st[L][NG][F];                               // S before token t0 + i
    float dvb[L][NG];                                   // dv of the block, stored after it
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int f = 0; f < F; ++f) st[0][g][f] = stn[g][f];
#pragma unroll
    for (int i = 0; i + 1 < L; ++i) fwd(st[i], st[i + 1], xn[i]);

#pragma unroll
    for (int i = L - 1; i >= 0; --i) {
      const int t = t0 + i;
      const bool ok = i < n;
      const size_t ti = tok(min(t, T - 1));
      Tok x;
      load_tok(x, t);
      float4 kx[F];
#pragma unroll
      for (int f = 0; f < F; ++f) kx[f] = cvt4(x.k[f]);
      float4 qq[F];
#pragma unroll
      for (int f = 0; f < F; ++f) qq[f] = load4(q + ti * DK + 64 * f + 4 * sub);
      floatx4 dq[F], dk[F];
#pragma unroll
      for (int f = 0; f < F; ++f) dq[f] = dk[f] = floatx4{0.f, 0.f, 0.f, 0.f};
      float da = 0.f, db = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float ddl = load1(dO + ti * dv + row0 + 4 * g);
        const float dd = ok ? ddl : 0.f;
        floatx4 sa[F], Gt[F];
#pragma unroll
        for (int f = 0; f < F; ++f) {
          sa[f] = st[i][g][f] * x.a;
          Gt[f] = floatx4{G[g][f][0] + dd * qq[f].x, G[g][f][1] + dd * qq[f].y,
                          G[g][f][2] + dd * qq[f].z, G[g][f][3] + dd * qq[f].w};
        }
        const float w = cvt1(x.v[g]) - sum16(dot4<F>(sa, kx));
        const float u = x.be * w;
        const float du = sum16(dot4<F>(Gt, kx));
        const float bdu = x.be * du;
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const float kf[4] = {kx[f].x, kx[f].y, kx[f].z, kx[f].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dq[f][e] += dd * (sa[f][e] + u * kf[e]);
            dk[f][e] += u * Gt[f][e] - bdu * sa[f][e];
            Gt[f][e] -= bdu * kf[e];                     // now dS~
          }
        }
        float pa = 0.f;
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
          for (int e = 0; e < 4; ++e) pa += Gt[f][e] * st[i][g][f][e];
        da += sum16(pa);
        db += du * w;
        dvb[i][g] = bdu;
#pragma unroll
        for (int f = 0; f < F; ++f) G[g][f] = Gt[f] * x.a;
      }
      // Over the wave's 4 row groups (lanes l, l^16, l^32, l^48 hold the
      // same columns), into the block's LDS partials (rows i >= n are
      // written but never read).  A reduce-scatter: at each of the two
      // exchange steps a lane sends the half of its values it gives away and
      // adds the partner's copy of the half it keeps (12 shuffles for the
      // 8 F dq and dk values instead of 16 F), and ends up owning one
      // quarter of the sums, which it stores: lane (h32, h16) holds dq
      // (h32 = 0) or dk (h32 = 1) at column 64 h16 + 4 sub .. + 3
      // (d_k = 128) or 4 sub + 2 h16 .. + 1 (d_k = 64).
      {
        constexpr int NV = 8 * F;
        float vals[NV];
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vals[4 * f + e] = dq[f][e];
            vals[4 * F + 4 * f + e] = dk[f][e];
          }
        const bool h32 = (lane & 32) != 0, h16 = (lane & 16) != 0;
        float v1[NV / 2], v2[NV / 4];
#pragma unroll
        for (int j = 0; j < NV / 2; ++j) {
          const float keep = h32 ? vals[NV / 2 + j] : vals[j];
          const float give = h32 ? vals[j] : vals[NV / 2 + j];
          v1[j] = keep + __shfl_xor(give, 32, 64);
        }
#pragma unroll
        for (int j = 0; j < NV / 4; ++j) {
          const float keep = h16 ? v1[NV / 4 + j] : v1[j];
          const float give = h16 ? v1[j] : v1[NV / 4 + j];
          v2[j] = keep + __shfl_xor(give, 16, 64);
        }
        float* dst = &red[i][wv][(h32 ? DK : 0) + (F == 2 ? 64 * h16 + 4 * sub : 4 * sub + 2 * h16)];
        if constexpr (F == 2) {
          *reinterpret_cast<floatx4*>(dst) = floatx4{v2[0], v2[1], v2[2], v2[3]};
        } else {
          *reinterpret_cast<float2*>(dst) = make_float2(v2[0], v2[1]);
        }
      }
      da = xsum_rows(da);
      db = xsum_rows(db);
      red2[i][wv][lane] = lane < 32 ? da : db;
    }
    prefetch(c - 1);
    __builtin_amdgcn_sched_barrier(0);                  // keep the loads ahead of the stores
    if (sub == 0) {
#pragma unroll
      for (int i = 0; i < L; ++i)
#pragma unroll
        for (int g = 0; g < NG; ++g)
          if (i < n) dv_out[tok(t0 + i) * dv + row0 + 4 * g] = dvb[i][g];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n * PW; e += 64 * kBwdWaves) {
      const int i = e / PW, j = e - i * PW;
      float x = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kBwdWaves; ++w2)
        x += j < 2 * DK ? red[i][w2][j] : red2[i][w2][j == 2 * DK ? 0 : 32];
      part[(((size_t)head * T + t0 + i) * wgs + wg) * PW + j] = x;
    }
    __syncthreads();                                    // red is reused by the next block
  }
  if (dS0) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int f = 0; f < F; ++f)
        *reinterpret_cast<floatx4*>(dS0 + srow(g) + 64 * f + 4 * sub) = G[g][f];
  }
}

// Sum of the workgroups' partials of each (head, token): one thread per
// output element, consecutive threads on consecutive elements.
template <int DK>
__global__ __launch_bounds__(256) void backward_reduce_kernel(
    const float* __restrict__ part, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dalpha, float* __restrict__ dbeta, long total, int H, int T,
    int wgs) {
  constexpr int PW = 2 * DK + 2;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const long ht = e / PW;
  const int j = (int)(e - ht * PW);
  const int head = (int)(ht / T), t = (int)(ht - (long)head * T);
  const int b = head / H, h = head - b * H;
  float x = 0.f;
  for (int w = 0; w < wgs; ++w) x += part[((size_t)ht * wgs + w) * PW + j];
  const size_t ti = ((size_t)b * T + t) * H + h;
  if (j < DK) dq[ti * DK + j] = x;
  else if (j < 2 * DK) dk[ti * DK + (j - DK)] = x;
  else if (j == 2 * DK) dalpha[ti] = x;
  else dbeta[ti] = x;
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, const void* dO,
                           const float* dST, float* dq, float* dk, float* dv_out,
                           float* dalpha, float* dbeta, float* dS0, int B, int T, int H,
                           int dkk, int dv, int in_dtype, float* ws, hipStream_t stream) {
  size_t ck = 0;
  backward_ws_floats(B, T, H, dkk, dv, &ck);
  float* ckpt = ws;
  float* part = ws + ck;
  const int wgs = backward_wgs(dkk, dv);
  const unsigned grid = (unsigned)((long)B * H * wgs);
#define GDN_BWD(DK, NG, TI)                                                                 \
  hipLaunchKernelGGL((backward_kernel<DK, NG, TI>), dim3(grid), dim3(64 * kBwdWaves), 0,   \
                     stream, static_cast<const TI*>(q), static_cast<const TI*>(k),         \
                     static_cast<const TI*>(v), alpha, beta, S0, static_cast<const TI*>(dO), \
                     dST, dv_out, dS0, ckpt, part, H, T, dv)
  const bool ib = in_dtype == 1;
  if (dkk == 128) {
    if (ib) GDN_BWD(128, 2, bf16);
    else GDN_BWD(128, 2, float);
  } else {
    if (ib) GDN_BWD(64, 2, bf16);
    else GDN_BWD(64, 2, float);
  }
#undef GDN_BWD
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  const long total = (long)B * H * T * backward_pw(dkk);
  const unsigned rgrid = (unsigned)((total + 255) / 256);
  if (dkk == 128)
    hipLaunchKernelGGL((backward_reduce_kernel<128>), dim3(rgrid), dim3(256), 0, stream, part, dq,
                       dk, dalpha, dbeta, total, H, T, wgs);
  else
    hipLaunchKernelGGL((backward_reduce_kernel<64>), dim3(rgrid), dim3(256), 0, stream, part, dq,
                       dk, dalpha, dbeta, total, H, T, wgs);
  return hipGetLastError();
}

}  // namespace gdn
