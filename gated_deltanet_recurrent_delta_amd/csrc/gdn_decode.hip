// Decode step of the gated delta rule: one token for a batch of carried
// fp32 states, fused into a single streaming pass over each state row.
//
// Per state row s_i (value channel i, dk floats) of a head:
//     p   = s_i . k          r  = s_i . q
//     u_i = beta (v_i - alpha p)                 (error of the decayed state)
//     s_i' = alpha s_i + u_i k                   (decay + delta write)
//     o_i  = s_i' . q = alpha r + u_i (k . q)    (readout of the new state)
// which is the per-row form of S' = alpha S (I - beta k k^T) + beta v k^T,
// o = S' q ("On State Reduction in Linear Attention", paper Sec. 2.1, Eq. (2) with
// the gated decay; rows evolve independently, paper Sec. 3.1).
//
// The step is HBM-bound (each state byte is read once and written once, at
// 0.75 flop/byte), so the kernel is a coalesced stream.  16 lanes cover 64
// columns of a row with 16-byte loads: at dk=64 one wave instruction reads
// four whole consecutive rows (1 KB), at dk=128 the first or second halves
// of four rows.  A wave issues its few vector loads (k, q, v) first and then
// every state load.  Two store orders, chosen at launch by the grid:
//   - streaming: each group of four rows is reduced and stored as soon as
//     its loads have arrived, so stores start while later rows are still in
//     flight (dk=128, and small batches);
//   - paced (dk=64 with at least 16 waves of 32 rows per CU): every row is
//     formed first, then the wave stores one 1 KB group at a time and waits
//     for each store to complete before issuing the next.  Measured on
//     MI355X at B=64, H=16, dv=128 (random states, fresh q/k/v per step),
//     this keeps 4096 waves' reads ahead of their writes and moves the
//     32 MiB state 4 % faster than the streaming order (11.8-11.9 against
//     12.3-12.6 us per step in one job).
// The optional input path (per-head channel subset of dk_in-wide q/k rows,
// L2 normalisation over the kept channels, query scale; "On State Reduction
// in Linear Attention", paper Sec. 3.2-3.3) is applied to k and q in
// registers before the row loop.  The two row dot products are reduced with
// four DPP steps and the state is read and written with non-temporal
// accesses.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// DK: key width; NG: groups of 4 rows per wave (rows per wave = 4 NG);
// WPB: waves per workgroup; PACED: the paced store order (see above).
// QK: the input path of a channel-pruned layer: 0 none (q, k used as
// given), 1 L2 normalisation (if qa.l2norm) and query scale, 2 the same
// after keeping the channels qa.chan[h][0 .. DK-1] of dk_in-wide rows.
template <int DK, int NG, int WPB, bool PACED, typename TIn, typename TOut, int QK>
__global__ __launch_bounds__(64 * WPB) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* S_in, float* S_out,
    TOut* __restrict__ o, int BH, int dv, int slices_per_head, int H,
    QkArgs qa) {
  constexpr int F = DK / 64;            // float4 per lane per row
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * WPB + (threadIdx.x >> 6);
  const int head = wave / slices_per_head;
  if (head >= BH) return;
  const int slice = wave - head * slices_per_head;
  const int sub = lane & 15;            // column lane within the row
  const int rg = lane >> 4;             // row within a group of 4
  const int row0 = slice * (4 * NG);

  // Loads: k and q first (with a channel subset, the indices and then the
  // kept channels), v and the gates, then the state rows, so that k and q
  // arrive first and each group of rows can be reduced and stored as soon
  // as its own loads are in.  (Issuing the gathered k/q loads after the
  // state loads instead measured slower: 13.97 against 13.75 us at B=64,
  // dk=64 from 128-wide rows.)
  float4 kk[F], qq[F];
  if constexpr (QK == 2) {
    const int* ch = qa.chan + (size_t)(head % H) * DK;
    const TIn* kr = k + (size_t)head * qa.dk_in;
    const TIn* qr = q + (size_t)head * qa.dk_in;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      int4 c = *reinterpret_cast<const int4*>(ch + 64 * f + 4 * sub);
      // an index outside the row is clamped into it: never an out-of-bounds read
      c.x = min(max(c.x, 0), qa.dk_in - 1);
      c.y = min(max(c.y, 0), qa.dk_in - 1);
      c.z = min(max(c.z, 0), qa.dk_in - 1);
      c.w = min(max(c.w, 0), qa.dk_in - 1);
      kk[f] = make_float4(load1(kr + c.x), load1(kr + c.y), load1(kr + c.z), load1(kr + c.w));
      qq[f] = make_float4(load1(qr + c.x), load1(qr + c.y), load1(qr + c.z), load1(qr + c.w));
    }
  } else {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      kk[f] = load4(k + (size_t)head * DK + 64 * f + 4 * sub);
      qq[f] = load4(q + (size_t)head * DK + 64 * f + 4 * sub);
    }
  }
  const float a = alpha[head];
  const float b = beta[head];
  float vv[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) vv[g] = load1(v + (size_t)head * dv + row0 + 4 * g + rg);

  const size_t sbase = (size_t)head * dv * DK;
  floatx4 s[NG][F];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float* rowp = S_in + sbase + (size_t)(row0 + 4 * g + rg) * DK;
#pragma unroll
    for (int f = 0; f < F; ++f)
      s[g][f] = __builtin_nontemporal_load(
          reinterpret_cast<const floatx4*>(rowp + 64 * f + 4 * sub));
  }

  // input path: normalise k and q over the kept channels (the 16 lanes of
  // a row hold all DK of them), scale q
  if constexpr (QK != 0) {
    // Branch-free: the norms are always formed and then selected, and the
    // reciprocal square root is the hardware one (1 ulp), so the kernel has
    // no branch here.  With a run-time branch (and the correctly rounded
    // 1/sqrt, a branchy sequence) the compiler hoisted the v loads above the
    // state loads, and the step took 12.5 instead of 11.9 us at B=64,
    // dk=64 (the plain instance's time), with or without normalisation.
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      sk += kk[f].x * kk[f].x + kk[f].y * kk[f].y + kk[f].z * kk[f].z + kk[f].w * kk[f].w;
      sq += qq[f].x * qq[f].x + qq[f].y * qq[f].y + qq[f].z * qq[f].z + qq[f].w * qq[f].w;
    }
    sk = sum16(sk);
    sq = sum16(sq);
    const bool nrm = qa.l2norm != 0;
    const float nk = nrm ? (sk > 0.f ? __builtin_amdgcn_rsqf(sk) : 0.f) : 1.f;
    const float nq = (nrm ? (sq > 0.f ? __builtin_amdgcn_rsqf(sq) : 0.f) : 1.f) * qa.qscale;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      kk[f].x *= nk; kk[f].y *= nk; kk[f].z *= nk; kk[f].w *= nk;
      qq[f].x *= nq; qq[f].y *= nq; qq[f].z *= nq; qq[f].w *= nq;
    }
  }

  float kq = 0.f;
#pragma unroll
  for (int f = 0; f < F; ++f)
    kq += kk[f].x * qq[f].x + kk[f].y * qq[f].y + kk[f].z * qq[f].z +
          kk[f].w * qq[f].w;
  kq = sum16(kq);

  float ov[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float p = 0.f, r = 0.f;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      p += s[g][f][0] * kk[f].x + s[g][f][1] * kk[f].y + s[g][f][2] * kk[f].z +
           s[g][f][3] * kk[f].w;
      r += s[g][f][0] * qq[f].x + s[g][f][1] * qq[f].y + s[g][f][2] * qq[f].z +
           s[g][f][3] * qq[f].w;
    }
    p = sum16(p);
    r = sum16(r);
    const float u = b * (vv[g] - a * p);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      s[g][f][0] = a * s[g][f][0] + u * kk[f].x;
      s[g][f][1] = a * s[g][f][1] + u * kk[f].y;
      s[g][f][2] = a * s[g][f][2] + u * kk[f].z;
      s[g][f][3] = a * s[g][f][3] + u * kk[f].w;
    }
    ov[g] = a * r + u * kq;
    if constexpr (!PACED) {
      const int row = row0 + 4 * g + rg;
      float* rowp = S_out + sbase + (size_t)row * DK;
#pragma unroll
      for (int f = 0; f < F; ++f)
        __builtin_nontemporal_store(s[g][f],
                                    reinterpret_cast<floatx4*>(rowp + 64 * f + 4 * sub));
      if (sub == 0) store1(o + (size_t)head * dv + row, ov[g]);
    }
  }
  if constexpr (PACED) {
    // every row is formed before the first store: without this barrier the
    // scheduler moves each group's arithmetic between the waits, and the
    // step measured 12.3 instead of 11.8 us (B=64, H=16, dk=64, dv=128)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float* rowp = S_out + sbase + (size_t)(row0 + 4 * g + rg) * DK;
#pragma unroll
      for (int f = 0; f < F; ++f) {
        __builtin_nontemporal_store(s[g][f],
                                    reinterpret_cast<floatx4*>(rowp + 64 * f + 4 * sub));
        if (g + 1 < NG || f + 1 < F) wait_vmem();
      }
    }
    if (sub == 0) {
#pragma unroll
      for (int g = 0; g < NG; ++g) store1(o + (size_t)head * dv + row0 + 4 * g + rg, ov[g]);
    }
  }
}

template <int DK, int NG, int WPB, bool PACED, typename TIn, typename TOut>
static void launch_decode_g(hipStream_t stream, const void* q, const void* k,
                            const void* v, const float* alpha,
                            const float* beta, const float* S_in, float* S_out,
                            void* o, int BH, int H, int dv, const QkArgs& qa) {
  const int slices = dv / (4 * NG);
  const long waves = (long)BH * slices;
  const dim3 grid((unsigned)((waves + WPB - 1) / WPB));
#define GDN_DEC_K(M)                                                                \
  hipLaunchKernelGGL((decode_kernel<DK, NG, WPB, PACED, TIn, TOut, M>), grid,        \
                     dim3(64 * WPB), 0, stream, static_cast<const TIn*>(q),          \
                     static_cast<const TIn*>(k), static_cast<const TIn*>(v),         \
                     alpha, beta, S_in, S_out, static_cast<TOut*>(o), BH, dv,        \
                     slices, H, qa)
  if (qa.chan != nullptr) GDN_DEC_K(2);
  else if (qa.l2norm || qa.qscale != 1.f) GDN_DEC_K(1);
  else GDN_DEC_K(0);
#undef GDN_DEC_K
}

template <int DK, typename TIn, typename TOut>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta,
                                  const float* S_in, float* S_out, void* o,
                                  int BH, int H, int dv, const QkArgs& qa,
                                  hipStream_t stream) {
  // Rows per wave and store order, measured on MI355X at H=16, dv=128 over
  // 18 rotating state sets (one process, one GPU):
  //   - dk=128: four rows per wave, streaming stores, at every batch (B=64:
  //     22.7 us per step; 22.8 with the paced order, 23.3 with 8 rows
  //     paced, 23.5 with the 8-lanes-per-row mapping).
  //   - dk=64 with at least kPaced waves of 32 rows: the paced order, one
  //     wave per workgroup.  B=64 with zero-filled buffers: 11.70 us, against
  //     11.78 / 11.84 with 2 / 4 waves per workgroup, 12.55 for the same
  //     layout without the waits, 12.7 waiting after every second store,
  //     13.2 paced with 16 rows per wave, 14.0 with each XCD taking a
  //     contiguous eighth of the rows, and 12.22 for the streaming order
  //     with 16 rows per wave below.  With random states and fresh q/k/v
  //     per step: 11.8-11.9 us against 12.5-12.6 for the streaming order.
  //   - dk=64 with kFill waves of 16 rows: streaming, 16 rows per wave,
  //     so that every CU is full from the first dispatch; else 8 rows under
  //     the same test; else 4 rows, which gives the most waves at small
  //     batches (B=1: 2.13 us, against 2.36 with 16 rows).
  constexpr long kPaced = 4096;         // 16 resident waves on each of 256 CUs
  constexpr long kFill = 8192;          // 32 resident waves on each of 256 CUs
  // dv is 64 or 128 (checked by the entry point), so 4, 8, 16 and 32 rows
  // divide it.
  if constexpr (DK == 64) {
    if ((long)BH * dv / 32 >= kPaced) {
      launch_decode_g<DK, 8, 1, true, TIn, TOut>(stream, q, k, v, alpha, beta, S_in,
                                                 S_out, o, BH, H, dv, qa);
      return hipGetLastError();
    }
    if ((long)BH * dv / 16 >= kFill) {
      launch_decode_g<DK, 4, 4, false, TIn, TOut>(stream, q, k, v, alpha, beta, S_in,
                                                  S_out, o, BH, H, dv, qa);
      return hipGetLastError();
    }
    if ((long)BH * dv / 8 >= kFill) {
      launch_decode_g<DK, 2, 4, false, TIn, TOut>(stream, q, k, v, alpha, beta, S_in,
                                                  S_out, o, BH, H, dv, qa);
      return hipGetLastError();
    }
  }
  launch_decode_g<DK, 1, 4, false, TIn, TOut>(stream, q, k, v, alpha, beta, S_in, S_out,
                                              o, BH, H, dv, qa);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta,
                         const float* S_in, float* S_out, void* o, int BH,
                         int H, int dk, int dv, int in_dtype, int out_dtype,
                         const QkArgs& qa, hipStream_t stream) {
#define GDN_DEC_DT(DK, TI, TO)                                               \
  return launch_decode_t<DK, TI, TO>(q, k, v, alpha, beta, S_in, S_out, o,   \
                                     BH, H, dv, qa, stream)
  const bool ib = in_dtype == 1, ob = out_dtype == 1;
  if (dk == 128) {
    if (ib && ob) GDN_DEC_DT(128, bf16, bf16);
    if (ib && !ob) GDN_DEC_DT(128, bf16, float);
    if (!ib && ob) GDN_DEC_DT(128, float, bf16);
    GDN_DEC_DT(128, float, float);
  } else {
    if (ib && ob) GDN_DEC_DT(64, bf16, bf16);
    if (ib && !ob) GDN_DEC_DT(64, bf16, float);
    if (!ib && ob) GDN_DEC_DT(64, float, bf16);
    GDN_DEC_DT(64, float, float);
  }
#undef GDN_DEC_DT
}

}  // namespace gdn
